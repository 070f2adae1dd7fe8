"""g4attn_decode_noalloc (no workspace, the library's per-GPU scratch array)
against g4attn_decode through the C ABI: bit-exact with the same split
count, on consecutive calls of different sizes (the second smaller, so stale
scratch contents from the first must not leak into it)."""

import numpy as np
import pytest
import torch

from g4inputs import gen

pytestmark = pytest.mark.gpu

DEV = "cuda"
SCRATCH = 32 << 20


def _case(B, Hq, Hkv, D, lens, cap, same, seed):
    q = gen.normal_bf16((B, Hq, D), (7, 77, seed, 0), "cpu").to(DEV)
    kc = torch.full((B, Hkv, cap, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    vc = kc if same else torch.full_like(kc, float("nan"))
    for b, n in enumerate(lens):
        kc[b, :, :n] = gen.normal_bf16((Hkv, n, D), (7, 77, seed + 1 + b, 0), "cpu").to(DEV)
        if not same:
            vc[b, :, :n] = gen.normal_bf16((Hkv, n, D), (7, 77, seed + 500 + b, 0), "cpu").to(DEV)
    return q, kc, vc, torch.tensor(lens, dtype=torch.int32, device=DEV)


def _both(g4, desc, q, kc, vc, kv_len, max_len, splits_ref, splits_noalloc=0):
    B, Hq = q.shape[0], q.shape[1]
    o_ref = torch.empty_like(q)
    l_ref = torch.empty((B, Hq), dtype=torch.float32, device=DEV)
    g4.g4attn_decode(desc, q, kc, vc, kv_len, max_len, o_ref, lse=l_ref, num_splits=splits_ref)
    o = torch.empty_like(q)
    l_ = torch.empty((B, Hq), dtype=torch.float32, device=DEV)
    g4.g4attn_decode_noalloc(desc, q, kc, vc, kv_len, max_len, o, lse=l_, num_splits=splits_noalloc)
    torch.cuda.synchronize()
    return o_ref, l_ref, o, l_


@pytest.mark.parametrize("D,same", [(512, True), (512, False), (256, True)])
def test_noalloc_equals_decode_two_calls(gpu_lib, D, same):
    g4 = gpu_lib
    desc = g4.layer_desc(16, 2, D)
    # first call: larger batch and lengths; second: smaller
    for B, lens, cap, seed in ((6, [4000, 1, 2500, 777, 3333, 64], 4096, 10), (2, [300, 45], 320, 40)):
        q, kc, vc, kv_len = _case(B, 16, 2, D, lens, cap, same, seed)
        o_ref, l_ref, o, l_ = _both(g4, desc, q, kc, vc, kv_len, max(lens), 0)
        assert torch.equal(o, o_ref), f"B={B} out"
        assert torch.equal(l_, l_ref), f"B={B} lse"


def test_noalloc_sliding_ring_equals_decode(gpu_lib):
    g4 = gpu_lib
    w = 256
    desc = g4.layer_desc(8, 2, 256, window=w)
    q, kc, vc, _ = _case(3, 8, 2, 256, [w, w, w], w, False, 70)
    kv_len = torch.tensor([5000, 100, 256], dtype=torch.int32, device=DEV)
    o_ref, l_ref, o, l_ = _both(g4, desc, q, kc, vc, kv_len, 5000, 0)
    assert torch.equal(o, o_ref) and torch.equal(l_, l_ref)


def test_noalloc_explicit_splits_then_smaller_call(gpu_lib):
    """An explicit split count whose partial results fit the scratch array is
    bit-exact with g4attn_decode at that count, the largest such count
    included; a count that does not fit is refused; then a small call reuses
    the array."""
    g4 = gpu_lib
    B, Hq, Hkv, D = 32, 32, 4, 512
    desc = g4.layer_desc(Hq, Hkv, D, rotary_dims=128)
    rng = np.random.default_rng(3)
    lens = rng.integers(1000, 8192, size=B, endpoint=True).tolist()
    q, kc, _, kv_len = _case(B, Hq, Hkv, D, lens, 8192, True, 100)
    max_len = max(lens)
    # the workspace grows with the split count: the largest count that fits
    ns = max(n for n in range(1, 65) if g4.g4attn_decode_workspace_bytes(desc, B, max_len, n) <= SCRATCH)
    assert 1 < ns < 32
    for n in (ns, 3):
        o_ref, l_ref, o, l_ = _both(g4, desc, q, kc, kc, kv_len, max_len, n, n)
        assert torch.equal(o, o_ref) and torch.equal(l_, l_ref), f"splits={n}"
    # an explicit count that does not fit is refused, nothing launched
    with pytest.raises(g4.G4AttnError) as ei:
        g4.g4attn_decode_noalloc(desc, q, kc, kc, kv_len, max_len, torch.empty_like(q), num_splits=32)
    assert ei.value.status == g4.ERR_WORKSPACE
    # a smaller call afterwards
    q2, kc2, vc2, kv2 = _case(3, Hq, Hkv, D, [900, 17, 2000], 2048, False, 300)
    o_ref, l_ref, o, l_ = _both(g4, desc, q2, kc2, vc2, kv2, 2000, 0)
    assert torch.equal(o, o_ref) and torch.equal(l_, l_ref)
