"""Chunked prefill over caches (g4attn_prefill_chunk) against the fp64 oracle through the C ABI:
position offsets, padded rows, sliding and global layers, both head widths."""

import numpy as np
import pytest
import torch

from g4inputs import gen
from oracle import attention as oat
from tests._cmp import assert_parity

pytestmark = pytest.mark.gpu

DEV = "cuda"
f64 = gen.to_f64
SENTINEL = 0x7FC3  # NaN pattern the padding rows must keep


def _bf(shape, seed):
    return gen.normal_bf16(shape, (7, 88, seed, 0), "cpu").to(DEV)


def _caches(B, Hkv, cap, D, total, seed):
    kc = torch.full((B, Hkv, cap, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    vc = torch.full_like(kc, float("nan"))
    for b, n in enumerate(total):
        kc[b, :, :n] = _bf((Hkv, n, D), seed + 2 * b)
        vc[b, :, :n] = _bf((Hkv, n, D), seed + 2 * b + 1)
    return kc, vc


@pytest.mark.parametrize("D,w,Hq,Hkv", [(256, 64, 8, 2), (256, 0, 4, 1), (512, 0, 8, 1), (512, 100, 8, 2)])
def test_prefill_chunk_vs_oracle(gpu_lib, D, w, Hq, Hkv):
    g4 = gpu_lib
    total = [300, 150, 97]          # positions each sequence holds so far, this chunk's included
    pos0 = [220, 100, 17]
    qlen = [80, 50, 80]
    B, S, cap = 3, 80, 320
    kc, vc = _caches(B, Hkv, cap, D, total, 40)
    q = _bf((B, S, Hq, D), 50)
    out = torch.full((B, S, Hq, D), SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=DEV)
    desc = g4.layer_desc(Hq, Hkv, D, window=w, rotary_dims=D)
    p0 = torch.tensor(pos0, dtype=torch.int32, device=DEV)
    ql = torch.tensor(qlen, dtype=torch.int32, device=DEV)
    g4.g4attn_prefill_chunk(desc, q, kc, vc, out, p0, ql, max(p + n - 1 for p, n in zip(pos0, qlen)), lse=lse)
    torch.cuda.synchronize()
    ro, rl = oat.prefill_over_cache(f64(q), f64(kc), f64(vc), pos0, qlen, desc.scale, w)
    got = np.concatenate([f64(out[b, :qlen[b]]).ravel() for b in range(B)])
    ref = np.concatenate([ro[b, :qlen[b]].ravel() for b in range(B)])
    assert_parity(got, ref, f"chunk D={D} w={w} Hq={Hq} Hkv={Hkv}")
    for b in range(B):
        np.testing.assert_allclose(lse[b, :, :qlen[b]].cpu().numpy(), rl[b, :, :qlen[b]], rtol=0, atol=2e-3)
        assert bool((out[b, qlen[b]:].view(torch.int16) == SENTINEL).all()), f"padding rows of sequence {b} written"


@pytest.mark.parametrize("D,w", [(256, 48), (512, 0)])
def test_prefill_chunks_equal_whole_prefill(gpu_lib, D, w):
    """Three chunks over caches give the rows of one whole-sequence prefill (to the parity bar)."""
    g4 = gpu_lib
    B, Sfull, Hq, Hkv, chunk = 2, 300, 8, 2, 100
    q = _bf((B, Sfull, Hq, D), 60)
    k = _bf((B, Sfull, Hkv, D), 61)
    v = _bf((B, Sfull, Hkv, D), 62)
    desc = g4.layer_desc(Hq, Hkv, D, window=w, rotary_dims=D)
    whole = torch.empty_like(q)
    g4.g4attn_prefill(desc, q, k, v, whole)
    kc = k.permute(0, 2, 1, 3).contiguous()
    vc = v.permute(0, 2, 1, 3).contiguous()
    parts = torch.empty_like(q)
    ql = torch.full((B,), chunk, dtype=torch.int32, device=DEV)
    for c0 in range(0, Sfull, chunk):
        p0 = torch.full((B,), c0, dtype=torch.int32, device=DEV)
        qq = q[:, c0:c0 + chunk].contiguous()
        oo = torch.empty_like(qq)
        g4.g4attn_prefill_chunk(desc, qq, kc, vc, oo, p0, ql, c0 + chunk - 1)
        parts[:, c0:c0 + chunk] = oo
    torch.cuda.synchronize()
    assert_parity(f64(parts), f64(whole), f"chunks vs whole D={D} w={w}")
    # and both against the oracle on the last chunk
    ro, _ = oat.attention_band(f64(q), f64(k), f64(v), desc.scale, w, rows=np.arange(200, 300))
    assert_parity(f64(parts[:, 200:]), ro, f"last chunk vs oracle D={D} w={w}")


@pytest.mark.parametrize("D,w", [(256, 0), (256, 96), (512, 0)])
def test_prefill_chunk_reference_overflow_redo(gpu_lib, D, w):
    """The extended variant's recompute pass: chunked rows whose logits grow far past their
    first tile's maximum (q = e_0, k_j = j/2 e_0, scale 1), with bidirectional spans too."""
    g4 = gpu_lib
    B, Hq, Hkv, total, chunk = 1, 8, 1, 300, 100
    P = total - chunk
    q = torch.zeros((B, chunk, Hq, D), dtype=torch.bfloat16, device=DEV)
    q[..., 0] = 1.0
    j = torch.arange(total, device=DEV, dtype=torch.float32)
    kc = torch.zeros((B, Hkv, total, D), dtype=torch.bfloat16, device=DEV)
    kc[0, 0, :, 0] = (0.5 * j).to(torch.bfloat16)
    vc = _bf((B, Hkv, total, D), 70)
    desc = g4.layer_desc(Hq, Hkv, D, window=w, scale=1.0)
    lo, hi = gen.image_spans(total, [(230, 40)])
    slo = torch.from_numpy(lo[P:][None]).to(DEV)
    shi = torch.from_numpy(hi[P:][None]).to(DEV)
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, chunk), dtype=torch.float32, device=DEV)
    g4.g4attn_prefill_chunk(desc, q, kc, vc, out, torch.tensor([P], dtype=torch.int32, device=DEV),
                            torch.tensor([chunk], dtype=torch.int32, device=DEV), total - 1, lse=lse,
                            span_lo=slo, span_hi=shi)
    torch.cuda.synchronize()
    qf = torch.zeros((B, total, Hq, D), dtype=torch.float64)
    qf[:, P:] = torch.from_numpy(f64(q))
    kf = f64(kc).transpose(0, 2, 1, 3)
    vf = f64(vc).transpose(0, 2, 1, 3)
    m = oat.mask_spans(total, w, lo, hi)
    ro, rl = oat.attention_masked(qf.numpy(), kf, vf, 1.0, m)
    assert_parity(f64(out), ro[:, P:], f"chunk redo D={D} w={w}")
    np.testing.assert_allclose(lse.cpu().numpy(), rl[:, :, P:], rtol=1e-4, atol=2e-3)


@pytest.mark.parametrize("D,w", [(256, 64), (512, 0)])
def test_prefill_chunk_padded_batch_equals_single_bit_exact(gpu_lib, D, w):
    """A padded batch of chunks equals each sequence's chunk computed alone, bit for bit
    (gemma4-pt-claude README, "Tests": batched rows match each prompt on its own)."""
    g4 = gpu_lib
    total = [300, 150, 97]
    pos0 = [220, 100, 17]
    qlen = [80, 50, 80]
    B, S, cap, Hq, Hkv = 3, 80, 320, 8, 2
    kc, vc = _caches(B, Hkv, cap, D, total, 140)
    q = _bf((B, S, Hq, D), 150)
    desc = g4.layer_desc(Hq, Hkv, D, window=w, rotary_dims=D)
    out = torch.full((B, S, Hq, D), SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    lse = torch.zeros((B, Hq, S), dtype=torch.float32, device=DEV)
    g4.g4attn_prefill_chunk(desc, q, kc, vc, out, torch.tensor(pos0, dtype=torch.int32, device=DEV),
                            torch.tensor(qlen, dtype=torch.int32, device=DEV), 299, lse=lse)
    for b in range(B):
        o1 = torch.full((1, S, Hq, D), SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)
        l1 = torch.zeros((1, Hq, S), dtype=torch.float32, device=DEV)
        g4.g4attn_prefill_chunk(desc, q[b:b + 1], kc[b:b + 1], vc[b:b + 1], o1,
                                torch.tensor([pos0[b]], dtype=torch.int32, device=DEV),
                                torch.tensor([qlen[b]], dtype=torch.int32, device=DEV), 299, lse=l1)
        assert torch.equal(out[b:b + 1].view(torch.int16), o1.view(torch.int16)), f"sequence {b}"
        assert torch.equal(lse[b:b + 1, :, :qlen[b]], l1[:, :, :qlen[b]]), f"sequence {b} lse"


def _random_chunk_configs(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        D = int(rng.choice([256, 512]))
        Hkv = int(rng.choice([1, 2]))
        G = int(rng.choice([1, 2, 8]))
        w = int(rng.choice([0, 0, 1, 17, 64]))
        B = int(rng.integers(1, 4))
        total = [int(rng.integers(1, 300)) for _ in range(B)]
        pos0 = [int(rng.integers(0, t)) for t in total]
        # the chunk reaches the end of the cache, or stops short (its tail is then padding)
        qlen = [t - p if rng.integers(0, 2) else int(rng.integers(1, t - p + 1)) for t, p in zip(total, pos0)]
        out.append((B, G * Hkv, Hkv, D, w, tuple(total), tuple(pos0), tuple(qlen)))
    return out


@pytest.mark.parametrize("B,Hq,Hkv,D,w,total,pos0,qlen", _random_chunk_configs(20, 11))
def test_prefill_chunk_random_configs_vs_oracle(gpu_lib, B, Hq, Hkv, D, w, total, pos0, qlen):
    """Seeded random chunks: offsets, chunk lengths (down to one row), padding, windows and head
    groupings drawn together; padding rows stay untouched."""
    g4 = gpu_lib
    S = max(qlen)
    cap = max(total) + 8
    kc, vc = _caches(B, Hkv, cap, D, total, 500 + cap)
    q = _bf((B, S, Hq, D), 600 + S)
    out = torch.full((B, S, Hq, D), SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=DEV)
    desc = g4.layer_desc(Hq, Hkv, D, window=w, rotary_dims=D)
    g4.g4attn_prefill_chunk(desc, q, kc, vc, out, torch.tensor(pos0, dtype=torch.int32, device=DEV),
                            torch.tensor(qlen, dtype=torch.int32, device=DEV),
                            max(p + n - 1 for p, n in zip(pos0, qlen)), lse=lse)
    torch.cuda.synchronize()
    ro, rl = oat.prefill_over_cache(f64(q), f64(kc), f64(vc), list(pos0), list(qlen), desc.scale, w)
    got = np.concatenate([f64(out[b, :qlen[b]]).ravel() for b in range(B)])
    ref = np.concatenate([ro[b, :qlen[b]].ravel() for b in range(B)])
    assert_parity(got, ref, f"random chunk B={B} Hq={Hq} Hkv={Hkv} D={D} w={w} pos0={pos0} qlen={qlen}")
    for b in range(B):
        np.testing.assert_allclose(lse[b, :, :qlen[b]].cpu().numpy(), rl[b, :, :qlen[b]], rtol=0, atol=2e-3)
        assert bool((out[b, qlen[b]:].view(torch.int16) == SENTINEL).all()), f"padding rows of sequence {b} written"
