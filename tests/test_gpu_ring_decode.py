"""Sliding-layer decode over rolling caches (ring mode of g4attn_norm_rope, window > 0 in
g4attn_decode), against the fp64 oracle through the C ABI."""

import numpy as np
import pytest
import torch

from g4inputs import gen
from oracle import attention as oat
from oracle import norm_rope as onr
from tests._cmp import assert_parity

pytestmark = pytest.mark.gpu

DEV = "cuda"
f64 = gen.to_f64
POISON = 0x7FC1  # a quiet-NaN bf16 pattern in never-written slots


def _bf(shape, seed):
    return gen.normal_bf16(shape, (7, 77, seed, 0), "cpu").to(DEV)


def test_norm_rope_ring_placement_bit_exact(gpu_lib):
    """Ring writes land in slot p mod w, keep only the last w positions of a call, and leave
    other slots alone; each slot equals the linear-mode output of its position bit for bit."""
    g4 = gpu_lib
    B, H, D, w = 2, 3, 256, 64
    total = 205
    x = _bf((B, total, H, D), 1)
    wt = gen.norm_weight(D, (7, 77, 2, 0)).to(DEV)
    lin = torch.empty_like(x)
    g4.g4attn_norm_rope(x, lin, wt, D, D, 1e4)                       # positions 0..total-1
    ring = torch.full((B, H, w, D), POISON, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    done = 0
    for S in (40, 100, 1, 64):                                           # calls of S new positions
        pos0 = torch.full((B,), done, dtype=torch.int32, device=DEV)
        g4.g4attn_norm_rope(x[:, done:done + S].contiguous(), ring, wt, D, D, 1e4, pos0=pos0,
                            max_pos=done + S - 1, cache_cap=w, ring=True)
        done += S
        torch.cuda.synchronize()
        pos = oat.ring_positions(done, w)
        for s in range(w):
            if pos[s] >= 0:
                assert torch.equal(ring[:, :, s], lin[:, pos[s]]), (done, s)
            else:
                assert bool((ring[:, :, s].view(torch.int16) == POISON).all()), (done, s)
    assert done == total


def _ring_case(g4, B, Hq, Hkv, D, w, lens, splits, seed):
    """Post-prologue query and rolling K/V caches filled with positions 0..n_b-1 (slot p mod w)."""
    q = _bf((B, Hq, D), seed)
    kfull = _bf((B, Hkv, max(lens), D), seed + 1)
    vfull = _bf((B, Hkv, max(lens), D), seed + 2)
    kr = torch.full((B, Hkv, w, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    vr = torch.full((B, Hkv, w, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    for b, n in enumerate(lens):
        pos = oat.ring_positions(n, w)
        slots = torch.as_tensor(np.nonzero(pos >= 0)[0], device=DEV)
        src = torch.as_tensor(pos[pos >= 0], device=DEV)
        kr[b][:, slots] = kfull[b][:, src]
        vr[b][:, slots] = vfull[b][:, src]
    desc = g4.layer_desc(Hq, Hkv, D, window=w, rotary_dims=D, rope_theta=1e4)
    kv_len = torch.tensor(lens, dtype=torch.int32, device=DEV)
    out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=DEV)
    g4.g4attn_decode(desc, q, kr, vr, kv_len, max(lens), out, lse=lse, num_splits=splits)
    torch.cuda.synchronize()
    return q, kr, vr, out, lse, desc


@pytest.mark.parametrize("Hq,Hkv,D,w", [(8, 1, 256, 512), (4, 2, 256, 64), (8, 2, 512, 128)])
@pytest.mark.parametrize("splits", [0, 1, 3])
def test_sliding_decode_ring_vs_oracle(gpu_lib, Hq, Hkv, D, w, splits):
    g4 = gpu_lib
    lens = [1, w - 1, w, w + 1, 3 * w + 7, 17]
    q, kr, vr, out, lse, desc = _ring_case(g4, len(lens), Hq, Hkv, D, w, lens, splits, 10 + splits)
    ro, rl = oat.sliding_decode_ring(f64(q), f64(kr), f64(vr), np.array(lens), desc.scale, w)
    assert_parity(f64(out), ro, f"ring decode Hq={Hq} Hkv={Hkv} D={D} w={w} splits={splits}")
    np.testing.assert_allclose(lse.cpu().numpy(), rl, rtol=0, atol=2e-3)


def test_sliding_decode_equals_uncached_forward(gpu_lib):
    """Prologue into rolling caches + decode of the last token, against the oracle's sliding
    prefill row computed from the raw inputs (the forward pass without a cache)."""
    g4 = gpu_lib
    Hq, Hkv, D, w, theta = 8, 2, 256, 128, 1e4
    lens = [50, 128, 129, 700]
    B = len(lens)
    S = max(lens)
    qx, kx, vx = _bf((B, S, Hq, D), 30), _bf((B, S, Hkv, D), 31), _bf((B, S, Hkv, D), 32)
    wq = gen.norm_weight(D, (7, 77, 33, 0)).to(DEV)
    wk = gen.norm_weight(D, (7, 77, 34, 0)).to(DEV)
    kr = torch.empty((B, Hkv, w, D), dtype=torch.bfloat16, device=DEV)
    vr = torch.empty_like(kr)
    qd = torch.empty((B, 1, Hq, D), dtype=torch.bfloat16, device=DEV)
    for b, n in enumerate(lens):
        zero = torch.zeros(1, dtype=torch.int32, device=DEV)
        # the sequence's keys/values so far (positions 0..n-1) into its ring, in one call
        g4.g4attn_norm_rope(kx[b:b + 1, :n].contiguous(), kr[b:b + 1], wk, D, D, theta, pos0=zero,
                            max_pos=n - 1, cache_cap=w, ring=True)
        g4.g4attn_norm_rope(vx[b:b + 1, :n].contiguous(), vr[b:b + 1], None, D, 0, theta, pos0=zero,
                            max_pos=n - 1, cache_cap=w, ring=True)
        pos = torch.full((1,), n - 1, dtype=torch.int32, device=DEV)
        g4.g4attn_norm_rope(qx[b:b + 1, n - 1:n].contiguous(), qd[b:b + 1], wq, D, D, theta, pos0=pos,
                            max_pos=n - 1)
    desc = g4.layer_desc(Hq, Hkv, D, window=w, rotary_dims=D, rope_theta=theta)
    out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=DEV)
    g4.g4attn_decode(desc, qd.view(B, Hq, D), kr, vr, torch.tensor(lens, dtype=torch.int32, device=DEV), S, out)
    torch.cuda.synchronize()
    ref = []
    for b, n in enumerate(lens):
        posn = np.arange(n)[None, :]
        q = onr.norm_rope(f64(qx[b:b + 1, :n]), f64(wq), posn, D, theta)
        k = onr.norm_rope(f64(kx[b:b + 1, :n]), f64(wk), posn, D, theta)
        v = onr.norm_rope(f64(vx[b:b + 1, :n]), None, posn, 0, theta)
        ro, _ = oat.attention_band(q, k, v, desc.scale, w, rows=np.array([n - 1]))
        ref.append(ro[0, 0])
    assert_parity(f64(out), np.stack(ref), "ring decode vs uncached forward")
