"""Pins for the fp64 attention oracle; CPU only."""

import numpy as np
import pytest
import torch

from oracle import attention as at

RNG = np.random.default_rng(99)


def _qkv(B, S, Hq, Hkv, D, scale_in=1.0):
    q = RNG.standard_normal((B, S, Hq, D)) * scale_in
    k = RNG.standard_normal((B, S, Hkv, D)) * scale_in
    v = RNG.standard_normal((B, S, Hkv, D))
    return q, k, v


def _sdpa_ref(q, k, v, scale, window):
    """torch SDPA (float64, CPU) with a mask built from torch.tril."""
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)
    kt = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(Hq // Hkv, dim=1)
    vt = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(Hq // Hkv, dim=1)
    ones = torch.ones(S, S, dtype=torch.bool)
    mask = torch.tril(ones)
    if window:
        mask = mask & ~torch.tril(ones, diagonal=-window)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    s = scale * (qt @ kt.transpose(-1, -2))
    s = s.masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    return o.permute(0, 2, 1, 3).numpy(), lse.numpy()


CASES = [
    # B, S, Hq, Hkv, D, window
    (1, 1, 2, 1, 16, 0), (1, 2, 2, 2, 16, 0), (2, 3, 4, 2, 8, 1), (1, 15, 8, 1, 16, 4),
    (1, 16, 8, 1, 16, 16), (1, 17, 8, 1, 16, 16), (1, 63, 2, 1, 32, 4), (1, 64, 2, 2, 16, 0),
    (2, 65, 4, 2, 16, 16), (1, 33, 8, 1, 256, 8), (1, 40, 4, 1, 512, 0),
]


@pytest.mark.parametrize("B,S,Hq,Hkv,D,w", CASES)
def test_band_equals_bruteforce(B, S, Hq, Hkv, D, w):
    q, k, v = _qkv(B, S, Hq, Hkv, D)
    scale = 1.0 / np.sqrt(D)
    o1, l1, wts = at.attention_bruteforce(q, k, v, scale, w)
    o2, l2 = at.attention_band(q, k, v, scale, w, block=7)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-12)
    # every row of the weights sums to one
    np.testing.assert_allclose(wts.sum(-1), 1.0, rtol=0, atol=1e-12)
    # a subset of rows gives the same rows
    rows = np.unique(np.array([0, S // 2, S - 1]))
    o3, l3 = at.attention_band(q, k, v, scale, w, rows=rows)
    np.testing.assert_allclose(o3, o1[:, rows], rtol=0, atol=1e-12)
    np.testing.assert_allclose(l3, l1[:, :, rows], rtol=0, atol=1e-12)


@pytest.mark.parametrize("B,S,Hq,Hkv,D,w", CASES)
def test_matches_torch_sdpa(B, S, Hq, Hkv, D, w):
    q, k, v = _qkv(B, S, Hq, Hkv, D)
    scale = 1.0 / np.sqrt(D)
    o, l_ = at.attention_band(q, k, v, scale, w)
    ro, rl = _sdpa_ref(q, k, v, scale, w)
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l_, rl, rtol=0, atol=1e-12)


def test_gqa_grouping_matches_torch_enable_gqa():
    q, k, v = _qkv(1, 20, 8, 2, 16)
    o, _ = at.attention_band(q, k, v, 0.25, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).permute(0, 2, 1, 3), torch.from_numpy(k).permute(0, 2, 1, 3),
        torch.from_numpy(v).permute(0, 2, 1, 3), is_causal=True, scale=0.25, enable_gqa=True)
    np.testing.assert_allclose(o, ref.permute(0, 2, 1, 3).numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("S,w", [(1, 0), (10, 0), (10, 1), (10, 3), (700, 512), (5000, 1024), (4096, 0)])
def test_visible_count_closed_form(S, w):
    cnt = at.visible_count(S, w)
    i = np.arange(S)
    expect = i + 1 if w == 0 else np.minimum(i + 1, w)
    np.testing.assert_array_equal(cnt, expect)
    # closed form of the total: w(w+1)/2 + (S-w)w past the window, else S(S+1)/2
    total = S * (S + 1) // 2 if (w == 0 or S <= w) else w * (w + 1) // 2 + (S - w) * w
    assert at.visible_pairs(S, w) == total
    if S <= 64:
        np.testing.assert_array_equal(at.mask_bruteforce(S, w).sum(1), expect)


def test_workload_pair_counts():
    # visible pairs per head at the workload shapes (enumerated mask) against
    # the hand-computed closed forms: 512*513/2 + 512*512, 8192*8193/2,
    # 1024*1025/2 + 15360*1024, 32768*32769/2
    assert at.visible_pairs(1024, 512) == 393472
    assert at.visible_pairs(8192, 0) == 33558528
    assert at.visible_pairs(16384, 1024) == 16253440
    assert at.visible_pairs(32768, 0) == 536887296


@pytest.mark.parametrize("S,w,images", [(40, 8, [(3, 5), (20, 12)]), (64, 0, [(0, 10), (30, 34)]),
                                        (300, 64, [(0, 20), (40, 150), (250, 50)])])
def test_visible_count_with_spans_matches_the_mask(S, w, images):
    lo, hi = at.span_rows(S, images)
    cnt = at.visible_count(S, w, lo, hi, block=7)
    np.testing.assert_array_equal(cnt, at.mask_spans(S, w, lo, hi).sum(axis=1))
    if S <= 64:   # and the element-by-element mask with the span rule written out
        m = at.mask_bruteforce(S, w)
        for i in range(S):
            for j in range(S):
                m[i, j] |= bool(lo[i] <= j <= hi[i])
        np.testing.assert_array_equal(cnt, m.sum(axis=1))


def test_window_one_gives_v_and_short_sequences_equal_global():
    q, k, v = _qkv(1, 30, 4, 2, 16)
    o, l_ = at.attention_band(q, k, v, 0.3, 1)
    np.testing.assert_array_equal(o, np.repeat(v, 2, axis=2))
    # S <= w: sliding == global, bit-identical
    og, lg = at.attention_band(q, k, v, 0.3, 0)
    for w in (30, 31, 512):
        ow, lw = at.attention_band(q, k, v, 0.3, w)
        np.testing.assert_array_equal(ow, og)
        np.testing.assert_array_equal(lw, lg)


def test_zero_scale_lse_counts_visible_keys():
    q, k, v = _qkv(1, 50, 2, 1, 8)
    for w in (0, 1, 7, 64):
        _, l_ = at.attention_band(q, k, v, 0.0, w)
        np.testing.assert_allclose(np.exp(l_[0, 0]), at.visible_count(50, w), rtol=1e-13)


def test_decode_equals_last_prefill_row_and_split_combine():
    B, S, Hq, Hkv, D = 2, 37, 8, 2, 32
    q, k, v = _qkv(B, S, Hq, Hkv, D)
    scale = 1.0 / np.sqrt(D)
    o, l_ = at.attention_band(q, k, v, scale, 0)
    kc = np.ascontiguousarray(k.transpose(0, 2, 1, 3))
    vc = np.ascontiguousarray(v.transpose(0, 2, 1, 3))
    for t in (0, 5, S - 1):
        od, ld = at.decode_attention(q[:, t], kc, vc, np.array([t + 1] * B), scale)
        np.testing.assert_allclose(od, o[:, t], rtol=0, atol=1e-12)
        np.testing.assert_allclose(ld, l_[:, :, t], rtol=0, atol=1e-12)
    # softmax over a union of disjoint key ranges = LSE-weighted combine of the parts
    n = np.array([S, S])
    full_o, full_l = at.decode_attention(q[:, -1], kc, vc, n, scale)
    cuts = [0, 5, 6, 20, S]
    parts = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        po, pl = at.decode_attention(q[:, -1], kc[:, :, a:b], vc[:, :, a:b], np.array([b - a] * B), scale)
        parts.append((po, pl))
    lse = np.logaddexp.reduce(np.stack([p[1] for p in parts]), axis=0)
    comb = sum(np.exp(pl - lse)[..., None] * po for po, pl in parts)
    np.testing.assert_allclose(lse, full_l, rtol=0, atol=1e-12)
    np.testing.assert_allclose(comb, full_o, rtol=0, atol=1e-12)


def test_decode_shared_cache_tensor():
    # K=V decode: one cache array used as both keys and values
    q = RNG.standard_normal((2, 8, 16))
    c = RNG.standard_normal((2, 1, 40, 16))
    o1, l1 = at.decode_attention(q, c, c, np.array([40, 17]), 0.25)
    o2, l2 = at.decode_attention(q, c, c.copy(), np.array([40, 17]), 0.25)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


# ----------------------------------------------- planted mistakes are caught
def test_planted_window_off_by_one_fails_count_pin():
    def wrong_visible(i, j, window):   # the primer's literal [i - w, i]: w + 1 keys
        d = i - j
        return (d >= 0) & (d <= window)
    i = np.arange(100)[:, None]
    j = np.arange(100)[None, :]
    assert not np.array_equal(wrong_visible(i, j, 16).sum(1), np.minimum(np.arange(100) + 1, 16))


def test_planted_gqa_mapping_fails_sdpa_pin():
    q, k, v = _qkv(1, 12, 4, 2, 8)
    ref, _ = _sdpa_ref(q, k, v, 0.3, 0)
    # interleaved grouping (h % Hkv) instead of contiguous (h // (Hq/Hkv))
    k2 = k[:, :, [0, 1, 0, 1]]
    v2 = v[:, :, [0, 1, 0, 1]]
    bad, _ = at.attention_band(q, k2, v2, 0.3, 0)
    assert not np.allclose(bad, ref, atol=1e-6)


@pytest.mark.parametrize("n,w", [(0, 8), (1, 8), (5, 8), (8, 8), (9, 8), (23, 8), (1000, 64), (64, 64)])
def test_ring_positions_closed_form(n, w):
    """Sequential writes to slot p mod w leave slot s holding p = L - ((L - s) mod w), L = n - 1."""
    pos = at.ring_positions(n, w)
    L = n - 1
    for s in range(w):
        want = L - ((L - s) % w) if n > 0 else -1
        assert pos[s] == (want if want >= 0 else -1)
    # the slots hold exactly the last min(n, w) positions
    assert sorted(p for p in pos if p >= 0) == list(range(max(0, n - w), n))


@pytest.mark.parametrize("S,w,Hq,Hkv", [(1, 16, 4, 1), (15, 16, 4, 1), (16, 16, 4, 2), (17, 16, 2, 2),
                                        (53, 16, 4, 2), (200, 32, 8, 1)])
def test_sliding_decode_ring_equals_uncached_forward(S, w, Hq, Hkv):
    """Decoding the last token over the rolling caches equals row S-1 of the sliding prefill."""
    D = 32
    q, k, v = _qkv(1, S, Hq, Hkv, D)
    scale = 1.0 / np.sqrt(D)
    pos = at.ring_positions(S, w)
    kr = np.full((1, Hkv, w, D), np.nan)
    vr = np.full((1, Hkv, w, D), np.nan)
    for s in range(w):
        if pos[s] >= 0:
            kr[0, :, s] = k[0, pos[s]]
            vr[0, :, s] = v[0, pos[s]]
    o, l_ = at.sliding_decode_ring(q[:, S - 1], kr, vr, np.array([S]), scale, w)
    ro, rl = at.attention_band(q, k, v, scale, w, rows=np.array([S - 1]))
    np.testing.assert_allclose(o, ro[:, 0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(l_, rl[:, :, 0], rtol=0, atol=1e-12)


def test_planted_ring_slot_off_by_one_fails_forward_pin():
    """A ring that places position p at slot (p + 1) mod w loses the pin against the forward pass."""
    S, w, D = 40, 16, 32
    q, k, v = _qkv(1, S, 2, 1, D)
    kr = np.zeros((1, 1, w, D))
    vr = np.zeros((1, 1, w, D))
    for p in range(S - w + 1, S):          # the last w-1 positions, shifted by one slot
        kr[0, 0, (p + 1) % w] = k[0, p, 0]
        vr[0, 0, (p + 1) % w] = v[0, p, 0]
    o, _ = at.sliding_decode_ring(q[:, S - 1], kr, vr, np.array([S]), 1.0 / np.sqrt(D), w)
    ro, _ = at.attention_band(q, k, v, 1.0 / np.sqrt(D), w, rows=np.array([S - 1]))
    assert np.abs(o - ro[:, 0]).max() > 1e-3


@pytest.mark.parametrize("w", [0, 5, 16])
def test_prefill_over_cache_equals_whole_sequence_rows(w):
    """Chunks of new rows over caches give the whole-sequence prefill's rows; padding stays empty."""
    B, S, Hq, Hkv, D = 3, 12, 4, 2, 16
    total = [40, 25, 12]        # positions of each sequence so far (cache rows)
    pos0 = np.array([28, 20, 0])
    qlen = np.array([12, 5, 9])  # row t < qlen[b] is position pos0[b] + t
    scale = 1.0 / np.sqrt(D)
    cap = 48
    kc = np.full((B, Hkv, cap, D), np.nan)
    vc = np.full((B, Hkv, cap, D), np.nan)
    qc = np.full((B, S, Hq, D), np.nan)
    refs = []
    for b in range(B):
        q, k, v = _qkv(1, total[b], Hq, Hkv, D)
        kc[b, :, :total[b]] = k[0].transpose(1, 0, 2)
        vc[b, :, :total[b]] = v[0].transpose(1, 0, 2)
        qc[b, :qlen[b]] = q[0, pos0[b]:pos0[b] + qlen[b]]
        rows = np.arange(pos0[b], pos0[b] + qlen[b])
        refs.append(at.attention_band(q, k, v, scale, w, rows=rows))
    o, l_ = at.prefill_over_cache(qc, kc, vc, pos0, qlen, scale, w)
    for b in range(B):
        np.testing.assert_allclose(o[b, :qlen[b]], refs[b][0][0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(l_[b, :, :qlen[b]], refs[b][1][0], rtol=0, atol=1e-12)
        assert np.all(o[b, qlen[b]:] == 0) and np.all(np.isneginf(l_[b, :, qlen[b]:]))


def test_span_mask_structure_and_degenerate_spans():
    S, w = 40, 8
    images = [(3, 5), (12, 14), (30, 10)]
    lo, hi = at.span_rows(S, images)
    m = at.mask_spans(S, w, lo, hi)
    plain = at.mask_bruteforce(S, w)
    for st, n in images:                 # inside a block: everything visible
        assert m[st:st + n, st:st + n].all()
    inside = np.zeros((S, S), bool)
    for st, n in images:
        inside[st:st + n, st:st + n] = True
    assert np.array_equal(m & ~inside, plain & ~inside)   # outside: the window mask
    dlo, dhi = at.span_rows(S, [])
    assert np.array_equal(at.mask_spans(S, w, dlo, dhi), plain)


@pytest.mark.parametrize("w", [0, 6])
def test_masked_oracle_matches_sdpa_and_band(w):
    B, S, Hq, Hkv, D = 1, 37, 4, 2, 16
    q, k, v = _qkv(B, S, Hq, Hkv, D)
    scale = 1.0 / np.sqrt(D)
    lo, hi = at.span_rows(S, [(2, 7), (20, 12)])
    m = at.mask_spans(S, w, lo, hi)
    o, l_ = at.attention_masked(q, k, v, scale, m)
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)
    kt = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(Hq // Hkv, dim=1)
    vt = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(Hq // Hkv, dim=1)
    ro = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(m), scale=scale)
    np.testing.assert_allclose(o, ro.permute(0, 2, 1, 3).numpy(), rtol=0, atol=1e-12)
    # degenerate spans: the band oracle
    dlo, dhi = at.span_rows(S, [])
    o2, l2 = at.attention_masked(q, k, v, scale, at.mask_spans(S, w, dlo, dhi))
    ob, lb = at.attention_band(q, k, v, scale, w)
    np.testing.assert_allclose(o2, ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2, lb, rtol=0, atol=1e-12)


def test_one_span_over_a_global_sequence_is_unmasked_attention():
    B, S, Hq, Hkv, D = 1, 20, 2, 1, 8
    q, k, v = _qkv(B, S, Hq, Hkv, D)
    lo, hi = at.span_rows(S, [(0, S)])
    o, _ = at.attention_masked(q, k, v, 0.3, at.mask_spans(S, 0, lo, hi))
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)
    kt = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(Hq // Hkv, dim=1)
    vt = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(Hq // Hkv, dim=1)
    ro = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=0.3)
    np.testing.assert_allclose(o, ro.permute(0, 2, 1, 3).numpy(), rtol=0, atol=1e-12)
