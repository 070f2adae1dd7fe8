"""Chunked prefill of a K=V global layer over its raw-projection cache (g4attn_kv_tied_append +
g4attn_prefill_chunk_tied), and bidirectional spans on the K=V whole-sequence prefill, against
the fp64 oracle through the C ABI."""

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
D, ROT, THETA = 512, 128, 1e6
SENTINEL = 0x7FC3  # NaN pattern the padding rows must keep


def _bf(shape, seed):
    return gen.normal_bf16(shape, (7, 123, seed, 0), "cpu").to(DEV)


def _cache(g4, X, wk, cap):
    """The layer's cache of positions 0 .. X.shape[1]-1 of every sequence (NaN past them)."""
    B, T, Hkv, _ = X.shape
    xc = torch.full((B, Hkv, cap, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    rc = torch.full((B, Hkv, cap), float("nan"), dtype=torch.float32, device=DEV)
    kc = torch.full((B, Hkv, cap, ROT), float("nan"), dtype=torch.bfloat16, device=DEV)
    g4.g4attn_kv_tied_append(X, wk, xc, rc, kc, THETA)
    return xc, rc, kc


def _oracle_kv(X, wk):
    """K, V caches [B, Hkv, T, D] of the oracle at positions 0 .. T-1."""
    B, T = X.shape[0], X.shape[1]
    K, V = onr.kv_tied_k_v(f64(X), f64(wk), np.tile(np.arange(T), (B, 1)), ROT, THETA)
    return K.transpose(0, 2, 1, 3), V.transpose(0, 2, 1, 3)


@pytest.mark.parametrize("Hq,Hkv,w", [(8, 1, 0), (16, 2, 0), (8, 2, 100), (16, 1, 0)])
def test_prefill_chunk_tied_vs_oracle(gpu_lib, Hq, Hkv, w):
    g4 = gpu_lib
    total = [300, 150, 97]          # positions each sequence holds so far, this chunk's included
    pos0 = [220, 100, 17]
    qlen = [80, 50, 80]
    B, S, cap = 3, 80, 320
    X = _bf((B, max(total), Hkv, D), 1 + Hkv)
    wk = gen.norm_weight(D, (7, 123, 2, 0)).to(DEV)
    xc, rc, kc = _cache(g4, X, wk, cap)
    q = _bf((B, S, Hq, D), 3 + Hkv)
    out = torch.full((B, S, Hq, D), SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=DEV)
    desc = g4.layer_desc(Hq, Hkv, D, window=w, k_eq_v=True, rotary_dims=ROT, rope_theta=THETA)
    p0 = torch.tensor(pos0, dtype=torch.int32, device=DEV)
    ql = torch.tensor(qlen, dtype=torch.int32, device=DEV)
    g4.g4attn_prefill_chunk_tied(desc, q, xc, rc, kc, wk, out, p0, ql, lse=lse)
    torch.cuda.synchronize()
    K, V = _oracle_kv(X, wk)
    ro, rl = oat.prefill_over_cache(f64(q), K, V, pos0, qlen, desc.scale, w)
    got = np.concatenate([f64(out[b, :qlen[b]]).ravel() for b in range(B)])
    ref = np.concatenate([ro[b, :qlen[b]].ravel() for b in range(B)])
    assert_parity(got, ref, f"K=V chunk Hq={Hq} Hkv={Hkv} w={w}")
    for b in range(B):
        # w_k and scale*log2(e) ride on q in bf16: up to ~2^-8 of a logit, as in the K=V decode test
        np.testing.assert_allclose(lse[b, :, :qlen[b]].cpu().numpy(), rl[b, :, :qlen[b]], rtol=0, atol=1e-2)
        assert bool((out[b, qlen[b]:].view(torch.int16) == SENTINEL).all()), f"padding rows of sequence {b} written"


def test_prefill_chunks_tied_equal_whole_prefill(gpu_lib):
    """Chunks appended to the layer's cache and attended over it give the rows of one whole-sequence
    K=V prefill (to the parity bar: the chunk path scales q, the whole path scales r)."""
    g4 = gpu_lib
    B, S, Hq, Hkv, chunk = 2, 700, 16, 2, 256
    X = _bf((B, S, Hkv, D), 10)
    q = _bf((B, S, Hq, D), 11)
    wk = gen.norm_weight(D, (7, 123, 12, 0)).to(DEV)
    desc = g4.layer_desc(Hq, Hkv, D, k_eq_v=True, rotary_dims=ROT, rope_theta=THETA)
    whole = torch.empty_like(q)
    g4.g4attn_prefill(desc, q, X, None, whole, w_k=wk)
    xc = torch.full((B, Hkv, S, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    rc = torch.full((B, Hkv, S), float("nan"), dtype=torch.float32, device=DEV)
    kc = torch.full((B, Hkv, S, ROT), float("nan"), dtype=torch.bfloat16, device=DEV)
    out = torch.empty_like(q)
    for c0 in range(0, S, chunk):
        n = min(chunk, S - c0)
        p0 = torch.full((B,), c0, dtype=torch.int32, device=DEV)
        ql = torch.full((B,), n, dtype=torch.int32, device=DEV)
        g4.g4attn_kv_tied_append(X[:, c0:c0 + n], wk, xc, rc, kc, THETA, pos0=p0, max_pos=c0 + n - 1)
        oo = torch.empty((B, n, Hq, D), dtype=torch.bfloat16, device=DEV)
        g4.g4attn_prefill_chunk_tied(desc, q[:, c0:c0 + n].contiguous(), xc, rc, kc, wk, oo, p0, ql,
                                     max_pos=c0 + n - 1)
        out[:, c0:c0 + n] = oo
    torch.cuda.synchronize()
    assert_parity(f64(out), f64(whole), "K=V chunks vs whole")


def test_prefill_chunk_tied_counts(gpu_lib):
    """scale = 0: every visible cached key weighs the same, so rint(exp(lse)) is each row's visible-key
    count, bit-exact, for every row and head (padded batch, window and global)."""
    g4 = gpu_lib
    total = [1000, 333, 64]
    pos0 = [700, 200, 0]
    qlen = [300, 133, 64]
    B, S, cap, Hq, Hkv = 3, 300, 1024, 8, 1
    X = _bf((B, max(total), Hkv, D), 20)
    wk = gen.norm_weight(D, (7, 123, 21, 0)).to(DEV)
    xc, rc, kc = _cache(g4, X, wk, cap)
    q = _bf((B, S, Hq, D), 22)
    for w in (0, 128):
        desc = g4.layer_desc(Hq, Hkv, D, window=w, k_eq_v=True, rotary_dims=ROT, rope_theta=THETA, scale=0.0)
        out = torch.empty_like(q)
        lse = torch.empty((B, Hq, S), dtype=torch.float32, device=DEV)
        g4.g4attn_prefill_chunk_tied(desc, q, xc, rc, kc, wk, out, torch.tensor(pos0, dtype=torch.int32,
                                     device=DEV), torch.tensor(qlen, dtype=torch.int32, device=DEV), lse=lse)
        torch.cuda.synchronize()
        for b in range(B):
            cnt = np.rint(np.exp(lse[b, :, :qlen[b]].double().cpu().numpy()))   # padding rows hold no lse
            want = oat.visible_count(total[b], w)[pos0[b]:pos0[b] + qlen[b]]
            assert np.array_equal(cnt, np.broadcast_to(want, (Hq, qlen[b]))), f"w={w} b={b}"


@pytest.mark.parametrize("Hq,Hkv", [(8, 1), (16, 2)])
def test_prefill_tied_spans_vs_oracle(gpu_lib, Hq, Hkv):
    """Bidirectional image spans on the K=V whole-sequence prefill."""
    g4 = gpu_lib
    B, S = 2, 300
    layouts = [[(0, 20), (40, 150), (250, 50)], [(31, 2), (63, 66), (140, 1)]]
    X = _bf((B, S, Hkv, D), 30 + Hkv)
    q = _bf((B, S, Hq, D), 32 + Hkv)
    wk = gen.norm_weight(D, (7, 123, 33, 0)).to(DEV)
    lo = np.stack([gen.image_spans(S, im)[0] for im in layouts])
    hi = np.stack([gen.image_spans(S, im)[1] for im in layouts])
    desc = g4.layer_desc(Hq, Hkv, D, k_eq_v=True, rotary_dims=ROT, rope_theta=THETA)
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=DEV)
    g4.g4attn_prefill(desc, q, X, None, out, w_k=wk, lse=lse, span_lo=torch.from_numpy(lo).to(DEV),
                      span_hi=torch.from_numpy(hi).to(DEV))
    torch.cuda.synchronize()
    K, V = onr.kv_tied_k_v(f64(X), f64(wk), np.tile(np.arange(S), (B, 1)), ROT, THETA)
    for b in range(B):
        m = oat.mask_spans(S, 0, lo[b], hi[b])
        ro, rl = oat.attention_masked(f64(q[b:b + 1]), K[b:b + 1], V[b:b + 1], desc.scale, m)
        assert_parity(f64(out[b:b + 1]), ro, f"K=V spans b={b}")
        np.testing.assert_allclose(lse[b:b + 1].cpu().numpy(), rl, rtol=0, atol=1e-2)


def _random_tied_chunk_configs(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        Hkv = int(rng.choice([1, 2, 4]))
        G = int(rng.choice([1, 4, 8]))
        w = int(rng.choice([0, 0, 33, 128]))
        B = int(rng.integers(1, 4))
        total = [int(rng.integers(1, 260)) for _ in range(B)]
        pos0 = [int(rng.integers(0, t)) for t in total]
        qlen = [t - p if rng.integers(0, 2) else int(rng.integers(1, t - p + 1)) for t, p in zip(total, pos0)]
        out.append((B, G * Hkv, Hkv, w, tuple(total), tuple(pos0), tuple(qlen)))
    return out


@pytest.mark.parametrize("B,Hq,Hkv,w,total,pos0,qlen", _random_tied_chunk_configs(20, 13))
def test_prefill_chunk_tied_random_configs(gpu_lib, B, Hq, Hkv, w, total, pos0, qlen):
    """Seeded random K=V chunks over the raw-projection cache: offsets, chunk lengths (down to one
    row), padding, windows and head groupings drawn together."""
    g4 = gpu_lib
    S, cap = max(qlen), max(total) + 8
    X = _bf((B, max(total), Hkv, D), 40 + cap)
    wk = gen.norm_weight(D, (7, 123, 41, 0)).to(DEV)
    xc, rc, kc = _cache(g4, X, wk, cap)
    q = _bf((B, S, Hq, D), 42 + S)
    out = torch.full((B, S, Hq, D), SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=DEV)
    desc = g4.layer_desc(Hq, Hkv, D, window=w, k_eq_v=True, rotary_dims=ROT, rope_theta=THETA)
    g4.g4attn_prefill_chunk_tied(desc, q, xc, rc, kc, wk, out, torch.tensor(pos0, dtype=torch.int32, device=DEV),
                                 torch.tensor(qlen, dtype=torch.int32, device=DEV), lse=lse)
    torch.cuda.synchronize()
    K, V = _oracle_kv(X, wk)
    ro, rl = oat.prefill_over_cache(f64(q), K, V, list(pos0), list(qlen), desc.scale, w)
    got = np.concatenate([f64(out[b, :qlen[b]]).ravel() for b in range(B)])
    ref = np.concatenate([ro[b, :qlen[b]].ravel() for b in range(B)])
    assert_parity(got, ref, f"random K=V chunk B={B} Hq={Hq} Hkv={Hkv} w={w} pos0={pos0} qlen={qlen}")
    for b in range(B):
        np.testing.assert_allclose(lse[b, :, :qlen[b]].cpu().numpy(), rl[b, :, :qlen[b]], rtol=0, atol=1e-2)
        assert bool((out[b, qlen[b]:].view(torch.int16) == SENTINEL).all()), f"padding rows of sequence {b} written"
