"""GPU parity: the HIP kernels (through the C ABI) against the fp64 oracle.

Shapes sweep tile boundaries and ragged tails; the bit-exact identities
(window 1, single key, pass-through RoPE dims, zero weight, mask counts,
rerun determinism) are checked exactly.
"""

import numpy as np
import pytest
import torch

from g4inputs import gen
from oracle import attention as oat
from oracle import norm_rope as onr
from tests._cmp import assert_parity

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _bf(shape, seed, scale=1.0):
    return gen.normal_bf16(shape, (7, 99, seed, 0), "cpu", scale).to(DEV)


def _w(D, seed):
    return gen.norm_weight(D, (7, 98, seed, 0)).to(DEV)


f64 = gen.to_f64


# ------------------------------------------------------------------ prologue
@pytest.mark.parametrize("D,rot,theta", [(256, 256, 1e4), (512, 128, 1e6), (512, 512, 1e6), (256, 0, 1e4)])
@pytest.mark.parametrize("weighted", [True, False])
def test_norm_rope_vs_oracle(gpu_lib, D, rot, theta, weighted):
    g4 = gpu_lib
    B, S, H = 2, 37, 3
    x = _bf((B, S, H, D), 1, 3.0)
    w = _w(D, 2) if weighted else None
    y = torch.empty_like(x)
    g4.g4attn_norm_rope(x, y, w, D, rot, theta)
    torch.cuda.synchronize()
    pos = np.tile(np.arange(S), (B, 1))
    ref = onr.norm_rope(f64(x), None if w is None else f64(w), pos, rot, theta)
    got = f64(y)
    # one rounding to bf16 of an fp32 computation: within 1 bf16 ulp everywhere
    ulp = np.maximum(np.abs(ref), 1e-30) * 2.0 ** -7
    assert np.all(np.abs(got - ref) <= ulp + 1e-5)
    assert_parity(got, ref, "norm_rope")


def test_norm_rope_exact_identities(gpu_lib):
    g4 = gpu_lib
    D, B, S, H = 512, 1, 70, 4
    x = _bf((B, S, H, D), 3)
    w = _w(D, 4)
    y_rope = torch.empty_like(x)
    y_none = torch.empty_like(x)
    g4.g4attn_norm_rope(x, y_rope, w, D, 128, 1e6)
    g4.g4attn_norm_rope(x, y_none, w, D, 0, 1e6)
    # pass-through dims of a partial rotation are bit-identical to no rotation
    assert torch.equal(y_rope[..., 64:256], y_none[..., 64:256])
    assert torch.equal(y_rope[..., 320:], y_none[..., 320:])
    # position 0 is the identity
    assert torch.equal(y_rope[:, 0], y_none[:, 0])
    # plain weight: w = 0 gives exact zeros
    z = torch.empty_like(x)
    g4.g4attn_norm_rope(x, z, torch.zeros(D, dtype=torch.bfloat16, device=DEV), D, 128, 1e6)
    assert torch.count_nonzero(z) == 0


def test_norm_rope_positions_and_cache_mode(gpu_lib):
    g4 = gpu_lib
    D, B, S, H, cap = 512, 3, 5, 4, 200
    x = _bf((B, S, H, D), 5)
    w = _w(D, 6)
    pos0 = torch.tensor([0, 17, 150], dtype=torch.int32, device=DEV)
    cache = torch.full((B, H, cap, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    g4.g4attn_norm_rope(x, cache, w, D, 128, 1e6, pos0=pos0, cache_cap=cap)
    y = torch.empty_like(x)
    g4.g4attn_norm_rope(x, y, w, D, 128, 1e6, pos0=pos0)
    torch.cuda.synchronize()
    p = pos0.cpu().numpy()
    ref = onr.norm_rope(f64(x), f64(w), p[:, None] + np.arange(S)[None, :], 128, 1e6)
    assert_parity(f64(y), ref, "norm_rope pos0")
    for b in range(B):
        rows = cache[b, :, p[b]:p[b] + S].permute(1, 0, 2)
        assert torch.equal(rows, y[b])
    # rows outside the written ranges stay untouched
    written = torch.zeros(cap, dtype=torch.bool)
    assert torch.isnan(cache[0, :, S:p[1]].float()).all()
    with pytest.raises(g4.G4AttnError):
        g4.g4attn_norm_rope(x, cache, w, D, 128, 1e6, pos0=pos0, max_pos=cap, cache_cap=cap)
    del written


@pytest.mark.parametrize("D,H", [(256, 1), (256, 5), (256, 12), (256, 33), (512, 1), (512, 3), (512, 6), (512, 9)])
def test_norm_rope_head_groups(gpu_lib, D, H):
    """Head counts that leave the last wave of a token with fewer heads than it holds."""
    g4 = gpu_lib
    B, S = 2, 9
    rot, theta = (D, 1e4) if D == 256 else (128, 1e6)
    wide = _bf((B, S, 2 * H, D), 70 + H, 2.0)
    x = wide[:, :, ::2]                      # strided heads
    w = _w(D, 71)
    y = torch.empty_like(x)
    g4.g4attn_norm_rope(x, y, w, D, rot, theta)
    y_contig = torch.empty_like(x)
    g4.g4attn_norm_rope(x.contiguous(), y_contig, w, D, rot, theta)
    torch.cuda.synchronize()
    assert torch.equal(y, y_contig)
    pos = np.tile(np.arange(S), (B, 1))
    ref = onr.norm_rope(f64(x), f64(w), pos, rot, theta)
    ulp = np.maximum(np.abs(ref), 1e-30) * 2.0 ** -7
    assert np.all(np.abs(f64(y) - ref) <= ulp + 1e-5)
    # cache mode: rows pos0[b] + t of [B, H, cap, D]; nothing else written
    cap = 40
    pos0 = torch.tensor([3, 20], dtype=torch.int32, device=DEV)
    cache = torch.full((B, H, cap, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    g4.g4attn_norm_rope(x, cache, w, D, rot, theta, pos0=pos0, cache_cap=cap)
    y_pos = torch.empty_like(x)
    g4.g4attn_norm_rope(x, y_pos, w, D, rot, theta, pos0=pos0)
    torch.cuda.synchronize()
    for b, p0 in enumerate(pos0.tolist()):
        assert torch.equal(cache[b, :, p0:p0 + S].permute(1, 0, 2), y_pos[b])
        keep = torch.ones(cap, dtype=torch.bool)
        keep[p0:p0 + S] = False
        assert torch.isnan(cache[b][:, keep].float()).all()


@pytest.mark.parametrize("D,H", [(256, 12), (512, 9), (256, 1)])
@pytest.mark.parametrize("weighted", [True, False])
def test_norm_rope_in_place_equals_out_of_place(gpu_lib, D, H, weighted):
    """x == y (equal strides) is allowed: several waves per token then write
    rows of one token while others read theirs."""
    g4 = gpu_lib
    B, S = 2, 33
    rot, theta = (D, 1e4) if D == 256 else (128, 1e6)
    x = _bf((B, S, H, D), 80 + H, 2.0)
    w = _w(D, 81) if weighted else None
    y = torch.empty_like(x)
    g4.g4attn_norm_rope(x, y, w, D, rot, theta)
    z = x.clone()
    g4.g4attn_norm_rope(z, z, w, D, rot, theta)
    torch.cuda.synchronize()
    assert torch.equal(z, y)


# ------------------------------------------------------------------ prefill
PREFILL_CASES = [
    # B, S, Hq, Hkv, D, window
    (1, 1, 8, 1, 256, 512), (1, 2, 2, 2, 256, 0), (1, 31, 8, 1, 256, 16), (1, 33, 2, 1, 256, 0),
    (2, 65, 4, 2, 256, 64), (1, 129, 8, 1, 256, 512), (1, 300, 2, 2, 256, 100), (1, 700, 8, 1, 256, 512),
    (1, 1, 8, 1, 512, 0), (1, 17, 8, 1, 512, 0), (2, 130, 4, 1, 512, 0), (1, 257, 8, 2, 512, 0),
    (1, 200, 32, 4, 512, 0), (1, 99, 32, 16, 256, 32), (1, 50, 3, 1, 256, 0), (1, 45, 6, 2, 512, 7),
    # 12B global layer (16 query heads on one KV head), E4B sliding layer (4 per KV head, window 512)
    (1, 90, 16, 1, 512, 0), (1, 70, 16, 1, 256, 33), (1, 150, 8, 2, 256, 512),
]


def _prefill_inputs(B, S, Hq, Hkv, D, seed=11):
    q = _bf((B, S, Hq, D), seed)
    k = _bf((B, S, Hkv, D), seed + 1)
    v = _bf((B, S, Hkv, D), seed + 2)
    return q, k, v


@pytest.mark.parametrize("B,S,Hq,Hkv,D,w", PREFILL_CASES)
def test_prefill_vs_oracle(gpu_lib, B, S, Hq, Hkv, D, w):
    g4 = gpu_lib
    q, k, v = _prefill_inputs(B, S, Hq, Hkv, D)
    desc = g4.layer_desc(Hq, Hkv, D, window=w)
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=DEV)
    g4.g4attn_prefill(desc, q, k, v, out, lse=lse)
    torch.cuda.synchronize()
    ro, rl = oat.attention_band(f64(q), f64(k), f64(v), desc.scale, w)
    assert_parity(f64(out), ro, f"prefill {B,S,Hq,Hkv,D,w}")
    np.testing.assert_allclose(lse.cpu().numpy(), rl, rtol=0, atol=2e-3)
    # rerun determinism (no atomics; fixed reduction order)
    out2 = torch.empty_like(q)
    g4.g4attn_prefill(desc, q, k, v, out2)
    assert torch.equal(out, out2)


@pytest.mark.parametrize("D", [256, 512])
def test_prefill_bit_exact_identities(gpu_lib, D):
    g4 = gpu_lib
    B, S, Hq, Hkv = 1, 150, 8, 2
    q, k, v = _prefill_inputs(B, S, Hq, Hkv, D, seed=21)
    out = torch.empty_like(q)
    # window 1: each row sees only itself -> out = v exactly
    g4.g4attn_prefill(g4.layer_desc(Hq, Hkv, D, window=1), q, k, v, out)
    assert torch.equal(out, v.repeat_interleave(Hq // Hkv, dim=2))
    # S = 1: a single key -> out = v_0 exactly
    o1 = torch.empty_like(q[:, :1])
    g4.g4attn_prefill(g4.layer_desc(Hq, Hkv, D), q[:, :1].contiguous(), k[:, :1].contiguous(),
                      v[:, :1].contiguous(), o1)
    assert torch.equal(o1, v[:, :1].repeat_interleave(Hq // Hkv, dim=2))
    # S <= w: sliding equals global, bit-identical
    og = torch.empty_like(q)
    ow = torch.empty_like(q)
    g4.g4attn_prefill(g4.layer_desc(Hq, Hkv, D, window=0), q, k, v, og)
    g4.g4attn_prefill(g4.layer_desc(Hq, Hkv, D, window=S), q, k, v, ow)
    assert torch.equal(og, ow)


@pytest.mark.parametrize("S,w,D,G", [(300, 0, 512, 8), (1000, 100, 256, 2), (777, 512, 256, 8), (95, 16, 512, 1)])
def test_prefill_mask_counts_bit_exact(gpu_lib, S, w, D, G):
    """scale = 0: every visible logit is 0, so exp(lse) counts the visible keys exactly."""
    g4 = gpu_lib
    q, k, v = _prefill_inputs(1, S, G, 1, D, seed=31)
    desc = g4.layer_desc(G, 1, D, window=w, scale=0.0)
    out = torch.empty_like(q)
    lse = torch.empty((1, G, S), dtype=torch.float32, device=DEV)
    g4.g4attn_prefill(desc, q, k, v, out, lse=lse)
    cnt = np.rint(np.exp(lse.cpu().numpy().astype(np.float64))).astype(np.int64)
    expect = oat.visible_count(S, w)
    for h in range(G):
        np.testing.assert_array_equal(cnt[0, h], expect)


def test_prefill_poisoned_tails(gpu_lib):
    """Data past S must not matter: NaN beyond the sequence leaves the output unchanged."""
    g4 = gpu_lib
    B, S, Hq, Hkv, D, pad = 1, 77, 8, 1, 512, 40
    q, k, v = _prefill_inputs(B, S + pad, Hq, Hkv, D, seed=41)
    ref = torch.empty_like(q[:, :S])
    g4.g4attn_prefill(g4.layer_desc(Hq, Hkv, D), q[:, :S], k[:, :S], v[:, :S], ref)
    k[:, S:] = float("nan")
    v[:, S:] = float("nan")
    q[:, S:] = float("nan")
    out = torch.empty_like(q[:, :S])
    g4.g4attn_prefill(g4.layer_desc(Hq, Hkv, D), q[:, :S], k[:, :S], v[:, :S], out)
    assert torch.isfinite(out.float()).all()
    assert torch.equal(out, ref)


@pytest.mark.parametrize("B,S,Hq,Hkv", [(1, 1, 8, 1), (1, 40, 8, 1), (1, 300, 32, 4), (2, 129, 16, 2),
                                     (1, 70, 15, 5), (2, 33, 6, 3), (1, 200, 16, 1), (2, 45, 16, 1)])
def test_prefill_kv_tied_vs_oracle(gpu_lib, B, S, Hq, Hkv):
    g4 = gpu_lib
    D, rot, theta = 512, 128, 1e6
    x_q = _bf((B, S, Hq, D), 51)
    X = _bf((B, S, Hkv, D), 52)
    w_q, w_k = _w(D, 53), _w(D, 54)
    q = torch.empty_like(x_q)
    g4.g4attn_norm_rope(x_q, q, w_q, D, rot, theta)
    desc = g4.layer_desc(Hq, Hkv, D, k_eq_v=True, rotary_dims=rot, rope_theta=theta)
    out = torch.empty_like(q)
    g4.g4attn_prefill(desc, q, X, None, out, w_k=w_k)
    torch.cuda.synchronize()
    pos = np.tile(np.arange(S), (B, 1))
    K, V = onr.kv_tied_k_v(f64(X), f64(w_k), pos, rot, theta)
    ro, _ = oat.attention_band(f64(q), K, V, desc.scale, 0)
    assert_parity(f64(out), ro, "prefill K=V")


# ------------------------------------------------------------------ decode
def _decode_case(g4, B, Hq, Hkv, D, lens, cap, same, splits, seed=61):
    q = _bf((B, Hq, D), seed)
    kc = torch.full((B, Hkv, cap, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    vc = kc if same else torch.full_like(kc, float("nan"))
    for b, n in enumerate(lens):
        kc[b, :, :n] = _bf((Hkv, n, D), seed + 1 + b)
        if not same:
            vc[b, :, :n] = _bf((Hkv, n, D), seed + 100 + b)
    kv_len = torch.tensor(lens, dtype=torch.int32, device=DEV)
    desc = g4.layer_desc(Hq, Hkv, D)
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=DEV)
    g4.g4attn_decode(desc, q, kc, vc, kv_len, max(lens), out, lse=lse, num_splits=splits)
    torch.cuda.synchronize()
    return q, kc, vc, out, lse, desc


@pytest.mark.parametrize("D,same", [(512, True), (512, False), (256, True), (256, False)])
@pytest.mark.parametrize("splits", [0, 1, 2, 7])
def test_decode_vs_oracle(gpu_lib, D, same, splits):
    g4 = gpu_lib
    lens = [1, 17, 300, 1029, 64]
    q, kc, vc, out, lse, desc = _decode_case(g4, 5, 16, 2, D, lens, 1100, same, splits)
    kcn, vcn = f64(kc), f64(vc)
    ro, rl = oat.decode_attention(f64(q), kcn, kcn if same else vcn, np.array(lens), desc.scale)
    assert_parity(f64(out), ro, f"decode D={D} same={same} splits={splits}")
    np.testing.assert_allclose(lse.cpu().numpy(), rl, rtol=0, atol=2e-3)
    # a single visible row returns that row exactly
    G = 8
    assert torch.equal(out[0], vc[0, :, 0].repeat_interleave(G, dim=0))


@pytest.mark.parametrize("D,splits", [(256, 1), (512, 1), (512, 3)])
def test_decode_clamped_lengths(gpu_lib, D, splits):
    """kv_len is clamped to [0, max_kv_len] on the device: a length of 0 (or
    below) gives zeros and lse = -inf, one past max_kv_len reads only
    max_kv_len rows; the other sequences are unaffected."""
    g4 = gpu_lib
    B, Hq, Hkv, cap, maxlen = 4, 8, 2, 200, 150
    lens = [0, 37, -5, maxlen + 9]
    q, kc, vc, out, lse, desc = _decode_case(g4, B, Hq, Hkv, D, [1, 37, 1, maxlen], cap, False, splits)
    kv_len = torch.tensor(lens, dtype=torch.int32, device=DEV)
    out.fill_(1.0)
    g4.g4attn_decode(desc, q, kc, vc, kv_len, maxlen, out, lse=lse, num_splits=splits)
    torch.cuda.synchronize()
    for b in (0, 2):
        assert torch.count_nonzero(out[b]) == 0
        assert torch.isneginf(lse[b]).all()
    for b, n in ((1, 37), (3, maxlen)):
        ro, rl = oat.decode_attention(f64(q[b:b + 1]), f64(kc[b:b + 1, :, :n]), f64(vc[b:b + 1, :, :n]), [n],
                                      desc.scale)
        assert_parity(f64(out[b:b + 1]), ro, f"clamped decode b={b}")
        np.testing.assert_allclose(lse[b:b + 1].cpu().numpy(), rl, rtol=0, atol=2e-3)


def test_decode_split_counts_agree_and_shared_cache(gpu_lib):
    g4 = gpu_lib
    lens = [2000, 4097, 33]
    outs = []
    for splits in (1, 2, 7, 0):
        *_, out, _, _ = _decode_case(g4, 3, 8, 1, 512, lens, 4100, True, splits)
        outs.append(out.float())
    for o in outs[1:]:
        assert (o - outs[0]).abs().max().item() < 1e-2
    # v_cache == k_cache gives the same result as a copy of it
    q, kc, _, out_same, _, desc = _decode_case(g4, 3, 8, 1, 512, lens, 4100, True, 0)
    out_copy = torch.empty_like(q)
    kv_len = torch.tensor(lens, dtype=torch.int32, device=DEV)
    g4.g4attn_decode(desc, q, kc, kc.clone(), kv_len, max(lens), out_copy)
    assert (out_copy.float() - out_same.float()).abs().max().item() < 1e-2


def test_decode_equals_prefill_row(gpu_lib):
    """Cached decode of row t over the prefill's keys reproduces prefill row t."""
    g4 = gpu_lib
    B, S, Hq, Hkv, D = 1, 300, 8, 1, 512
    q, k, v = _prefill_inputs(B, S, Hq, Hkv, D, seed=71)
    pre = torch.empty_like(q)
    g4.g4attn_prefill(g4.layer_desc(Hq, Hkv, D), q, k, v, pre)
    kc = k.permute(0, 2, 1, 3).contiguous()
    vc = v.permute(0, 2, 1, 3).contiguous()
    for t in (0, 31, 32, 299):
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=DEV)
        kl = torch.tensor([t + 1], dtype=torch.int32, device=DEV)
        g4.g4attn_decode(g4.layer_desc(Hq, Hkv, D), q[:, t].contiguous(), kc, vc, kl, t + 1, out)
        assert (out.float() - pre[:, t].float()).abs().max().item() < 2e-2


@pytest.mark.parametrize("D,w,kv_tied", [(256, 0, False), (512, 0, False), (256, 200, False), (512, 0, True)])
def test_prefill_reference_overflow_redo(gpu_lib, D, w, kv_tied):
    """Logits that grow along the sequence far past the first tile's maximum
    (q = e_0, k_j = j/2 e_0, scale 1) force the recomputation pass."""
    g4 = gpu_lib
    B, S, Hq, Hkv = 1, 300, 8, 1
    q = torch.zeros((B, S, Hq, D), dtype=torch.bfloat16, device=DEV)
    q[..., 0] = 1.0
    j = torch.arange(S, device=DEV, dtype=torch.float32)
    k = torch.zeros((B, S, Hkv, D), dtype=torch.bfloat16, device=DEV)
    k[0, :, 0, 0] = (0.5 * j).to(torch.bfloat16)
    v = _bf((B, S, Hkv, D), 81)
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=DEV)
    if not kv_tied:
        desc = g4.layer_desc(Hq, Hkv, D, window=w, scale=1.0)
        g4.g4attn_prefill(desc, q, k, v, out, lse=lse)
        ro, rl = oat.attention_band(f64(q), f64(k), f64(v), 1.0, w)
    else:
        # K=V: X ~ N(0,1) except coordinate 101 (not rotated) = j/128, unit
        # weights.  The norm keeps K_101 close to j/128, so the logits 80 K_101
        # rise by ~170 after the first tile, while values stay O(1).
        X = _bf((B, S, Hkv, D), 82)
        X[0, :, 0, 101] = (j / 128).to(torch.bfloat16)
        q2 = torch.zeros_like(q)
        q2[..., 101] = 80.0
        wk = torch.ones(D, dtype=torch.bfloat16, device=DEV)
        desc = g4.layer_desc(Hq, Hkv, D, k_eq_v=True, rotary_dims=128, rope_theta=1e6, scale=1.0)
        g4.g4attn_prefill(desc, q2, X, None, out, w_k=wk, lse=lse)
        K, V = onr.kv_tied_k_v(f64(X), f64(wk), np.tile(np.arange(S), (B, 1)), 128, 1e6)
        ro, rl = oat.attention_band(f64(q2), K, V, 1.0, 0)
    torch.cuda.synchronize()
    assert_parity(f64(out), ro, f"redo D={D} w={w} tied={kv_tied}")
    np.testing.assert_allclose(lse.cpu().numpy(), rl, rtol=1e-4, atol=2e-3)


@pytest.mark.parametrize("same", [True, False])
def test_decode_reference_overflow_redo(gpu_lib, same):
    """Logits growing along the cache (coordinate 0 = j/2048, q_0 = 2560) rise
    by ~200 within one chunk, forcing the decode recomputation pass."""
    g4 = gpu_lib
    B, Hq, Hkv, D, n = 2, 8, 1, 512, 4000
    q = torch.zeros((B, Hq, D), dtype=torch.bfloat16, device=DEV)
    q[..., 0] = 2560.0
    kc = _bf((B, Hkv, n, D), 91)
    kc[:, :, :, 0] = (torch.arange(n, device=DEV, dtype=torch.float32) / 2048).to(torch.bfloat16)
    vc = kc if same else _bf((B, Hkv, n, D), 92)
    kv_len = torch.tensor([n, n - 1000], dtype=torch.int32, device=DEV)
    desc = g4.layer_desc(Hq, Hkv, D)
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=DEV)
    g4.g4attn_decode(desc, q, kc, vc, kv_len, n, out, lse=lse, num_splits=1)
    torch.cuda.synchronize()
    k64 = f64(kc)
    ro, rl = oat.decode_attention(f64(q), k64, k64 if same else f64(vc), kv_len.cpu().numpy(), desc.scale)
    assert_parity(f64(out), ro, f"decode redo same={same}")
    np.testing.assert_allclose(lse.cpu().numpy(), rl, rtol=1e-5, atol=2e-3)


def _random_configs(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        D = int(rng.choice([256, 512]))
        Hkv = int(rng.choice([1, 2, 4]))
        G = int(rng.choice([1, 2, 3, 8]))
        S = int(rng.integers(1, 420))
        w = int(rng.choice([0, 0, 1, 17, 64, 300]))
        B = int(rng.integers(1, 3))
        out.append((B, S, G * Hkv, Hkv, D, w))
    return out


@pytest.mark.parametrize("B,S,Hq,Hkv,D,w", _random_configs(30, 2024))
def test_prefill_random_configs_vs_oracle(gpu_lib, B, S, Hq, Hkv, D, w):
    """Seeded random shapes: lengths, windows, head groupings and widths drawn together."""
    g4 = gpu_lib
    q, k, v = _bf((B, S, Hq, D), 900 + S), _bf((B, S, Hkv, D), 901 + S), _bf((B, S, Hkv, D), 902 + S)
    desc = g4.layer_desc(Hq, Hkv, D, window=w, rotary_dims=D)
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=DEV)
    g4.g4attn_prefill(desc, q, k, v, out, lse=lse)
    torch.cuda.synchronize()
    ro, rl = oat.attention_band(f64(q), f64(k), f64(v), desc.scale, w)
    assert_parity(f64(out), ro, f"random B={B} S={S} Hq={Hq} Hkv={Hkv} D={D} w={w}")
    np.testing.assert_allclose(lse.cpu().numpy(), rl, rtol=0, atol=2e-3)


# ------------------------------------------------------------------ batching
@pytest.mark.parametrize("D,w,kv_tied", [(256, 64, False), (512, 0, False), (512, 0, True), (256, 0, False)])
def test_prefill_batched_equals_single_bit_exact(gpu_lib, D, w, kv_tied):
    """Batched rows equal each sequence computed on its own, bit for bit
    (gemma4-pt-claude README, "Tests": batched rows match single prompts):
    no part of a sequence's computation depends on the batch around it."""
    g4 = gpu_lib
    B, S, Hq, Hkv = 3, 333, 16, 2
    q, k, v = _prefill_inputs(B, S, Hq, Hkv, D, seed=111)
    wk = _w(D, 112)
    desc = g4.layer_desc(Hq, Hkv, D, window=w, k_eq_v=kv_tied, rotary_dims=128 if kv_tied else D)
    vv = None if kv_tied else v
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=DEV)
    g4.g4attn_prefill(desc, q, k, vv, out, w_k=wk if kv_tied else None, lse=lse)
    for b in range(B):
        o1 = torch.empty_like(q[b:b + 1])
        l1 = torch.empty((1, Hq, S), dtype=torch.float32, device=DEV)
        g4.g4attn_prefill(desc, q[b:b + 1], k[b:b + 1], None if kv_tied else v[b:b + 1], o1,
                          w_k=wk if kv_tied else None, lse=l1)
        assert torch.equal(out[b:b + 1], o1), f"sequence {b}"
        assert torch.equal(lse[b:b + 1], l1), f"sequence {b} lse"


def test_decode_batched_equals_single_bit_exact(gpu_lib):
    """A decode batch equals each sequence decoded alone when the split
    partition is the same (explicit split count and length bound)."""
    g4 = gpu_lib
    lens = [700, 1, 2049, 1500]
    for same in (True, False):
        q, kc, vc, out, lse, desc = _decode_case(g4, len(lens), 16, 2, 512, lens, 2100, same, 3)
        for b, n in enumerate(lens):
            o1 = torch.empty_like(q[b:b + 1])
            l1 = torch.empty((1, 16), dtype=torch.float32, device=DEV)
            kl = torch.tensor([n], dtype=torch.int32, device=DEV)
            g4.g4attn_decode(desc, q[b:b + 1], kc[b:b + 1], kc[b:b + 1] if same else vc[b:b + 1], kl, max(lens),
                             o1, lse=l1, num_splits=3)
            assert torch.equal(out[b:b + 1], o1), f"same={same} sequence {b}"
            assert torch.equal(lse[b:b + 1], l1), f"same={same} sequence {b} lse"


@pytest.mark.parametrize("D,w,kv_tied", [(256, 64, False), (256, 0, False), (512, 0, False), (512, 0, True)])
def test_prefill_wide_kv_row_stride(gpu_lib, D, w, kv_tied):
    """K and V (or X) read through views whose key-row stride is 2^20 elements (2 MiB): the byte offset
    of key 2048 from key 0 is 2^32, past 32 bits, while each 32-key tile's offsets stay within them.
    The output must be bit-identical to the same call on contiguous copies (the kernels' arithmetic
    does not depend on where the rows are), which is itself checked against the oracle."""
    g4 = gpu_lib
    B, S, Hq, Hkv, W = 1, 2049, 2, 1, 1 << 20
    q = _bf((B, S, Hq, D), 71)
    kc, vc = _bf((B, S, Hkv, D), 72), _bf((B, S, Hkv, D), 73)
    big = torch.empty((S, W), dtype=torch.bfloat16, device=DEV)          # 4 GiB + 2 MiB
    big[:, :D] = kc[0, :, 0]
    big[:, D:2 * D] = vc[0, :, 0]
    strides = (S * W, W, D, 1)
    kw = big.as_strided((B, S, Hkv, D), strides, 0)
    vw = big.as_strided((B, S, Hkv, D), strides, D)
    desc = g4.layer_desc(Hq, Hkv, D, window=w, k_eq_v=kv_tied, rotary_dims=128 if kv_tied else D)
    wk = gen.norm_weight(D, (7, 66, 74, 0)).to(DEV) if kv_tied else None
    out_w, out_c = torch.empty_like(q), torch.empty_like(q)
    g4.g4attn_prefill(desc, q, kw, None if kv_tied else vw, out_w, w_k=wk)
    g4.g4attn_prefill(desc, q, kc, None if kv_tied else vc, out_c, w_k=wk)
    torch.cuda.synchronize()
    del big
    assert torch.equal(out_w, out_c), f"wide-stride rows differ D={D} w={w} K=V={kv_tied}"
    if kv_tied:
        K, V = onr.kv_tied_k_v(f64(kc), f64(wk), np.arange(S)[None, :], 128, desc.rope_theta)
    else:
        K, V = f64(kc), f64(vc)
    ro, _ = oat.attention_band(f64(q), K, V, desc.scale, w)
    assert_parity(f64(out_c), ro, f"wide-stride reference D={D} w={w} K=V={kv_tied}")


# ------------------------------------------------------------------ randomized decode
def _random_decode_configs(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        D = int(rng.choice([256, 512]))
        Hkv = int(rng.choice([1, 2, 4]))
        G = int(rng.choice([1, 2, 4, 8, 16]))
        B = int(rng.integers(1, 5))
        # lengths: random, plus the edges (one row, exact tile and chunk multiples)
        lens = [int(rng.choice([1, 16, 256, int(rng.integers(1, 1500))])) for _ in range(B)]
        cap = max(lens) + int(rng.integers(0, 40))
        same = bool(rng.integers(0, 2))
        splits = int(rng.choice([0, 1, 3]))
        out.append((B, G * Hkv, Hkv, D, tuple(lens), cap, same, splits))
    return out


@pytest.mark.parametrize("B,Hq,Hkv,D,lens,cap,same,splits", _random_decode_configs(25, 7))
def test_decode_random_configs_vs_oracle(gpu_lib, B, Hq, Hkv, D, lens, cap, same, splits):
    """Seeded random decode shapes: batch, head grouping, width, lengths (with their edge values),
    capacity, shared or separate caches and split count drawn together."""
    g4 = gpu_lib
    q, kc, vc, out, lse, desc = _decode_case(g4, B, Hq, Hkv, D, list(lens), cap, same, splits, seed=300 + cap)
    kcn = f64(kc)
    ro, rl = oat.decode_attention(f64(q), kcn, kcn if same else f64(vc), np.array(lens), desc.scale)
    assert_parity(f64(out), ro, f"random decode B={B} Hq={Hq} Hkv={Hkv} D={D} lens={lens} same={same}")
    np.testing.assert_allclose(lse.cpu().numpy(), rl, rtol=0, atol=2e-3)
