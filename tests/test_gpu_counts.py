"""Mask and length logic at the full workload shapes, bit-exact, for every row.

With a logit scale of 0 every visible logit is exactly 0, so the softmax
denominator l_i is the number of keys row i sees: an integer, exact in fp32,
and rint(exp(lse_i)) must equal the oracle's count for every row, head and
sequence.  An off-by-one in a window, length, span or split boundary moves
random-data outputs by only ~1/w or ~1/n, under the value tolerance, so these
counts are what pins the index logic at full size (vinija.ai Gemma 4 primer,
"Sliding-window attention" and "Global attention layers"; gemma4-pt-claude
README, "KV Cache").

The inputs are the bench's own workloads (same builders, seeded draws and
launch configuration); only the scale in the layer descriptor is 0.
"""

import numpy as np
import pytest
import torch

import bench
from g4inputs import WORKLOADS, gen
from oracle import attention as oat

pytestmark = pytest.mark.gpu


def _zero_scale(g4, c, k_eq_v=None):
    return g4.layer_desc(c.Hq, c.Hkv, c.D, window=c.window, k_eq_v=c.k_eq_v if k_eq_v is None else k_eq_v,
                         rotary_dims=c.rotary_dims, rope_theta=c.theta, scale=0.0)


def _counts(lse):
    """rint(exp(lse)) in fp64, as int64 (lse is the fp32 natural log)."""
    return np.rint(np.exp(lse.cpu().numpy().astype(np.float64))).astype(np.int64)


@pytest.mark.parametrize("name", ["e2b_sliding_prefill", "e2b_global_prefill", "31b_sliding_prefill",
                                  "31b_global_kv_prefill", "31b_sliding_image_prefill"])
def test_full_size_prefill_counts_every_row(gpu_lib, name):
    g4 = gpu_lib
    c = WORKLOADS[name]
    print(f"[counts] prefill {name}", flush=True)
    s = bench.build_prefill(torch, g4, gen, c)
    s["desc"] = _zero_scale(g4, c)
    lse = torch.empty((c.B, c.Hq, c.S), dtype=torch.float32, device="cuda")
    bench.run_prefill(g4, s, lse=lse)
    torch.cuda.synchronize()
    lo, hi = gen.image_spans(c.S, c.images) if c.images else (None, None)
    expect = oat.visible_count(c.S, c.window, lo, hi)
    got = _counts(lse)
    for b in range(c.B):
        for h in range(c.Hq):
            np.testing.assert_array_equal(got[b, h], expect, err_msg=f"{name} b={b} h={h}")
    assert torch.isfinite(s["out"].float()).all()


def test_full_size_chunk_prefill_counts_every_row(gpu_lib):
    """The 31B sliding chunk (last 4096 of 16384 positions over linear caches)."""
    g4 = gpu_lib
    c = WORKLOADS["31b_sliding_chunk_prefill"]
    s = bench.build_chunk(torch, g4, gen, c)
    lse = torch.empty((c.B, c.Hq, c.S), dtype=torch.float32, device="cuda")
    bench.run_chunk_pro(g4, s)
    g4.g4attn_prefill_chunk(_zero_scale(g4, c), s["q"], s["kc"], s["vc"], s["out"], s["pos0"], s["qlen"],
                            s["total"] - 1, lse=lse, workspace=s["ws"])
    torch.cuda.synchronize()
    # row t is position p0 + t of a sequence of `total` positions
    expect = oat.visible_count(s["total"], c.window)[s["p0"]:s["p0"] + c.S]
    got = _counts(lse)
    for b in range(c.B):
        for h in range(c.Hq):
            np.testing.assert_array_equal(got[b, h], expect, err_msg=f"chunk b={b} h={h}")


def test_full_size_kv_chunk_prefill_counts_every_row(gpu_lib):
    """The 31B K=V chunk (last 4096 of 32768 positions over the raw-projection cache)."""
    g4 = gpu_lib
    c = WORKLOADS["31b_global_kv_chunk_prefill"]
    s = bench.build_kv_chunk(torch, g4, gen, c)
    lse = torch.empty((c.B, c.Hq, c.S), dtype=torch.float32, device="cuda")
    bench.run_chunk_pro(g4, s)
    g4.g4attn_prefill_chunk_tied(_zero_scale(g4, c), s["q"], s["xc"], s["rc"], s["krc"], s["wk"], s["out"],
                                 s["pos0"], s["qlen"], s["total"] - 1, lse=lse, workspace=s["ws"])
    torch.cuda.synchronize()
    expect = oat.visible_count(s["total"], c.window)[s["p0"]:s["p0"] + c.S]
    got = _counts(lse)
    for b in range(c.B):
        for h in range(c.Hq):
            np.testing.assert_array_equal(got[b, h], expect, err_msg=f"K=V chunk b={b} h={h}")


@pytest.mark.parametrize("name", ["31b_global_kv_decode", "31b_sliding_decode"])
@pytest.mark.parametrize("splits", [0, 1, 7])
def test_full_size_decode_counts_every_sequence(gpu_lib, name, splits):
    """Every sequence and head sees exactly its n_b positions (global) or the
    min(n_b, w) filled slots of its ring (sliding), whatever the split count."""
    g4 = gpu_lib
    c = WORKLOADS[name]
    print(f"[counts] decode {name} splits={splits}", flush=True)
    s = bench.build_decode(torch, g4, gen, c)
    desc = _zero_scale(g4, c, k_eq_v=False)
    lse = torch.empty((c.B, c.Hq), dtype=torch.float32, device="cuda")
    bench.run_decode_pro(g4, s)
    g4.g4attn_decode(desc, s["q"].view(c.B, c.Hq, c.D), s["cache"], s["vcache"], s["kv_len"], s["max_len"],
                     s["out"], lse=lse, num_splits=splits)
    torch.cuda.synchronize()
    n = s["n"]
    if c.window:
        # the new token at position n-1 sees positions p with 0 <= (n-1) - p < w
        expect = np.array([int(oat.visible(nb - 1, np.arange(nb), c.window).sum()) for nb in n])
    else:
        expect = np.array([int(oat.visible(nb - 1, np.arange(nb), 0).sum()) for nb in n])
    got = _counts(lse)
    for h in range(c.Hq):
        np.testing.assert_array_equal(got[:, h], expect, err_msg=f"{name} splits={splits} h={h}")


def test_full_size_raw_kv_decode_counts_every_sequence(gpu_lib):
    """The K=V decode over the raw-projection cache: n_b rows for every sequence and head."""
    g4 = gpu_lib
    c = WORKLOADS["31b_global_kv_decode_raw"]
    s = bench.build_decode_raw(torch, g4, gen, c)
    desc = _zero_scale(g4, c)
    lse = torch.empty((c.B, c.Hq), dtype=torch.float32, device="cuda")
    bench.run_decode_pro(g4, s)
    g4.g4attn_decode_tied(desc, s["q"].view(c.B, c.Hq, c.D), s["xc"], s["rc"], s["krc"], s["wk"], s["kv_len"],
                          s["max_len"], s["out"], lse=lse)
    torch.cuda.synchronize()
    expect = np.array([int(oat.visible(nb - 1, np.arange(nb), 0).sum()) for nb in s["n"]])
    got = _counts(lse)
    for h in range(c.Hq):
        np.testing.assert_array_equal(got[:, h], expect, err_msg=f"raw decode h={h}")
