"""The hot path inside a captured HIP graph.

No entry point allocates, synchronises or records a memset (every flag and
partial is written by the kernels of the call itself), so a serving loop can
capture a step once and replay it.  Each graph below is replayed several
times with new inputs written in place and other eager work in between, and
every replay must equal the eager calls bit for bit.
"""

import pytest
import torch

from g4inputs import gen

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _fill(t, key):
    t.copy_(gen.normal_bf16(tuple(t.shape), key, DEV))


def _capture(step):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                   # warm-up on a side stream, as torch requires
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    return g


def test_decode_step_replays_in_a_graph(gpu_lib):
    """q prologue at the new positions + K=V decode over a shared cache (two chunks per sequence)."""
    g4 = gpu_lib
    B, Hq, Hkv, D, cap = 4, 32, 4, 512, 3000
    desc = g4.layer_desc(Hq, Hkv, D, k_eq_v=True, rotary_dims=128, rope_theta=1e6)
    cache = gen.normal_bf16((B, Hkv, cap, D), (7, 200, 1, 0), DEV)
    w = gen.norm_weight(D, (7, 200, 2, 0)).to(DEV)
    q_raw = torch.empty((B, 1, Hq, D), dtype=torch.bfloat16, device=DEV)
    q = torch.empty_like(q_raw)
    kv_len = torch.empty(B, dtype=torch.int32, device=DEV)
    pos0 = torch.empty(B, dtype=torch.int32, device=DEV)
    out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=DEV)
    splits = 2
    ws = torch.empty(g4.g4attn_decode_workspace_bytes(desc, B, cap, splits), dtype=torch.uint8, device=DEV)

    def step():
        g4.g4attn_norm_rope(q_raw, q, w, D, 128, 1e6, pos0=pos0, max_pos=cap - 1)
        g4.g4attn_decode(desc, q.view(B, Hq, D), cache, cache, kv_len, cap, out, lse=lse, num_splits=splits,
                         workspace=ws)

    def set_inputs(i):
        _fill(q_raw, (7, 201, i, 0))
        lens = torch.tensor([cap - 7 * i, 1 + 300 * i, 1500 + i, 64 * (i + 1)], dtype=torch.int32)
        kv_len.copy_(lens)
        pos0.copy_(lens - 1)

    set_inputs(0)
    graph = _capture(step)
    for i in range(1, 5):
        set_inputs(i)
        step()                                   # eager reference
        torch.cuda.synchronize()
        ref_out, ref_lse = out.clone(), lse.clone()
        out.zero_()
        lse.zero_()
        torch.matmul(torch.randn(256, 256, device=DEV), torch.randn(256, 256, device=DEV))  # unrelated work
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"replay {i}"
        assert torch.equal(lse, ref_lse), f"replay {i}"


def test_sliding_prefill_replays_in_a_graph(gpu_lib):
    """q/k/v prologues + sliding-window prefill (recompute check launch included)."""
    g4 = gpu_lib
    B, S, Hq, Hkv, D, win = 2, 700, 8, 2, 256, 256
    desc = g4.layer_desc(Hq, Hkv, D, window=win, rotary_dims=D, rope_theta=1e4)
    raw = {n: torch.empty((B, S, h, D), dtype=torch.bfloat16, device=DEV) for n, h in (("q", Hq), ("k", Hkv),
                                                                                        ("v", Hkv))}
    post = {n: torch.empty_like(t) for n, t in raw.items()}
    wq, wk = gen.norm_weight(D, (7, 210, 1, 0)).to(DEV), gen.norm_weight(D, (7, 210, 2, 0)).to(DEV)
    out = torch.empty_like(raw["q"])
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=DEV)
    ws = torch.empty(g4.g4attn_prefill_workspace_bytes(desc, B, S), dtype=torch.uint8, device=DEV)

    def step():
        g4.g4attn_norm_rope(raw["q"], post["q"], wq, D, D, 1e4, max_pos=S - 1)
        g4.g4attn_norm_rope(raw["k"], post["k"], wk, D, D, 1e4, max_pos=S - 1)
        g4.g4attn_norm_rope(raw["v"], post["v"], None, D, 0, 1e4, max_pos=S - 1)
        g4.g4attn_prefill(desc, post["q"], post["k"], post["v"], out, lse=lse, workspace=ws)

    def set_inputs(i):
        for j, t in enumerate(raw.values()):
            _fill(t, (7, 211, i, j))

    set_inputs(0)
    graph = _capture(step)
    for i in range(1, 4):
        set_inputs(i)
        step()
        torch.cuda.synchronize()
        ref_out, ref_lse = out.clone(), lse.clone()
        out.zero_()
        lse.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"replay {i}"
        assert torch.equal(lse, ref_lse), f"replay {i}"
