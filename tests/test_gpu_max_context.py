"""Parity at the longest contexts the pages give: 256K positions on the 31B
model, 128K on E2B ("Gemma 4" Keras docs and the vinija.ai Gemma 4 primer,
context windows by variant).

At S = 262144 the 31B global layer's q holds exactly 2^32 elements, so these
cases exercise every 64-bit offset of the prologue, prefill and decode
kernels, and the index logic over the whole length:
- the 31B K=V global and sliding prefills at 256K and the E2B global
  (separate K and V) and sliding prefills at 128K, run as the bench runs its
  workloads (prologue + attention), with sampled rows (tile edges deep in
  the sequence included) against the fp64 oracle, then with a logit scale of
  0, where rint(exp(lse)) must equal the visible-key count of every row and
  head exactly wherever fp32 can carry it (see EXACT_COUNT);
- the K=V and sliding chunked prefills of the last 4096 of 262144 positions
  over their caches (raw projection for K=V, linear K/V for sliding), sampled
  rows and counts as above;
- the K=V decode of two sequences whose new token is the 262144th position,
  sampled heads against the oracle, then the same counts at three split
  counts.
"""

import numpy as np
import pytest
import torch

import bench
from g4inputs import gen
from g4inputs.configs import MAX_CONTEXT
from oracle import attention as oat
from oracle import norm_rope as onr

from tests._cmp import assert_parity
from tests._rows import LSE_ATOL, prefill_oracle_rows, sample_tokens

pytestmark = pytest.mark.gpu

f64 = gen.to_f64


# The kernels write lse = (m + log2 l) * ln 2 in fp32.  Near l = 2^18 one ulp
# of lse is 9.5e-7, so an ulp of the hardware log2 plus the final rounding
# moves exp(lse) by up to ~0.47 of a key: rint(exp(lse)) then sits at the
# limit of what fp32 can resolve.  Counts up to 2^17 keep a margin of two and
# are checked exactly; larger ones to 4 ulp of lse (the rows there are also
# pinned by the sampled-row values).  Decode counts use partitions into
# power-of-two chunks, whose logarithms are exact.
EXACT_COUNT = 1 << 17


def _counts(lse):
    """rint(exp(lse)) in fp64, as int64 (lse is the fp32 natural log)."""
    return np.rint(np.exp(lse.cpu().numpy().astype(np.float64))).astype(np.int64)


def _expected_counts(S, window, rows):
    """Visible keys of every prefill row: i + 1, or min(i + 1, w) on a sliding
    layer (the oracle's mask in closed form, pinned against its enumeration
    in the oracle tests), checked here against the oracle's own mask
    predicate over all S keys on the sampled rows."""
    i = np.arange(S)
    expect = i + 1 if window == 0 else np.minimum(i + 1, window)
    j = np.arange(S)
    for t in rows:
        assert int(oat.visible(int(t), j, window).sum()) == expect[t]
    return expect


def _zero_scale(g4, c):
    return g4.layer_desc(c.Hq, c.Hkv, c.D, window=c.window, k_eq_v=c.k_eq_v, rotary_dims=c.rotary_dims,
                         rope_theta=c.theta, scale=0.0)


@pytest.mark.parametrize("name", ["31b_global_kv_prefill_256k", "31b_sliding_prefill_256k",
                                  "e2b_global_prefill_128k", "e2b_sliding_prefill_128k"])
def test_prefill_max_context_sampled_rows_and_counts(gpu_lib, name):
    g4 = gpu_lib
    c = MAX_CONTEXT[name]
    print(f"[max] {name}: inputs and run", flush=True)
    s = bench.build_prefill(torch, g4, gen, c)
    lse = torch.empty((c.B, c.Hq, c.S), dtype=torch.float32, device="cuda")
    bench.run_prefill(g4, s, lse=lse)
    torch.cuda.synchronize()
    assert torch.isfinite(lse).all()
    G = c.Hq // c.Hkv
    # 32-key tile edges far into the sequence
    deep = [t for t in (32767, 32768, 65535, 65536, 131071, 131072, 262111, 262112) if t < c.S]
    got_all, ref_all = [], []
    for g in sorted({0, c.Hkv - 1}):
        toks = np.union1d(sample_tokens(c.S, c.window, n_rand=4, seed=(c.cfg_id, 0, g)), deep)
        heads = sorted({g * G, g * G + G - 1})
        print(f"[max] {name}: oracle rows of KV group {g}", flush=True)
        ro, rl = prefill_oracle_rows(s, 0, g, toks, heads)
        ti = torch.as_tensor(toks, device="cuda")
        hi = torch.as_tensor(heads, device="cuda")
        got_all.append(f64(s["out"][0].index_select(0, ti).index_select(1, hi)))
        ref_all.append(ro)
        got_lse = lse[0].index_select(0, hi).index_select(1, ti).T.cpu().numpy()
        np.testing.assert_allclose(got_lse, rl, rtol=0, atol=LSE_ATOL, err_msg=f"{name} g={g} lse")
    assert_parity(np.concatenate([x.reshape(-1) for x in got_all]),
                  np.concatenate([x.reshape(-1) for x in ref_all]), f"{name} sampled rows")

    print(f"[max] {name}: counts", flush=True)
    s["desc"] = _zero_scale(g4, c)
    bench.run_prefill(g4, s, lse=lse)
    torch.cuda.synchronize()
    expect = _expected_counts(c.S, c.window, np.union1d(deep, [0, 1, 1023, 1024, 1025, c.S - 1]))
    got = _counts(lse)
    exact = expect <= EXACT_COUNT
    rel = np.abs(np.exp(lse[0].cpu().numpy().astype(np.float64)) / expect[None, :] - 1.0)
    for h in range(c.Hq):
        np.testing.assert_array_equal(got[0, h][exact], expect[exact], err_msg=f"{name} counts h={h}")
    assert np.all(rel[:, ~exact] <= 4 * 2.0 ** -23 * 12.5), f"{name} counts past 2^17: {rel[:, ~exact].max()}"


@pytest.mark.parametrize("name", ["31b_global_kv_chunk_256k", "31b_sliding_chunk_256k"])
def test_chunk_256k_sampled_rows_and_counts(gpu_lib, name):
    g4 = gpu_lib
    c = MAX_CONTEXT[name]
    print(f"[max] {name}: inputs and run", flush=True)
    s = (bench.build_kv_chunk if c.k_eq_v else bench.build_chunk)(torch, g4, gen, c)
    lse = torch.empty((c.B, c.Hq, c.S), dtype=torch.float32, device="cuda")

    def run(desc):
        bench.run_chunk_pro(g4, s)
        if c.k_eq_v:
            g4.g4attn_prefill_chunk_tied(desc, s["q"], s["xc"], s["rc"], s["krc"], s["wk"], s["out"], s["pos0"],
                                         s["qlen"], s["total"] - 1, lse=lse, workspace=s["ws"])
        else:
            g4.g4attn_prefill_chunk(desc, s["q"], s["kc"], s["vc"], s["out"], s["pos0"], s["qlen"],
                                    s["total"] - 1, lse=lse, workspace=s["ws"])
        torch.cuda.synchronize()

    run(s["desc"])
    G = c.Hq // c.Hkv
    p0, total = s["p0"], s["total"]
    got_all, ref_all = [], []
    for g in (0, c.Hkv - 1):
        print(f"[max] {name}: oracle rows of KV group {g}", flush=True)
        if c.k_eq_v:   # the oracle's keys and values from the raw rows the cache was built from
            X = gen.normal_bf16((c.B, total, c.Hkv, c.D), gen.seed_key(c.cfg_id, gen.X), "cuda")
            K, V = onr.kv_tied_k_v(f64(X[0:1, :, g:g + 1]), f64(s["wk"]), np.arange(total)[None, :],
                                   c.rotary_dims, c.theta)
            del X
            kk_all, vv_all = K[0, :, 0], V[0, :, 0]
        toks = sample_tokens(c.S, 0, n_rand=4, seed=(c.cfg_id, 0, g))
        heads = [g * G, g * G + G - 1]
        for t in toks:
            p = p0 + int(t)
            k0 = 0 if c.window == 0 else p - c.window + 1
            if c.k_eq_v:
                kk, vv = kk_all[k0:p + 1], vv_all[k0:p + 1]
            else:
                kk, vv = f64(s["kc"][0, g, k0:p + 1]), f64(s["vc"][0, g, k0:p + 1])
            q = onr.norm_rope(f64(s["q_raw"][0:1, t:t + 1, heads]), f64(s["wq"]), np.array([[p]]), c.rotary_dims,
                              c.theta)
            for hi_, h in enumerate(heads):
                sc = c.scale * (kk @ q[0, 0, hi_])
                m = sc.max()
                e = np.exp(sc - m)
                ref_all.append((e @ vv) / e.sum())
                got_all.append(f64(s["out"][0, t, h]))
                np.testing.assert_allclose(float(lse[0, h, t]), m + np.log(e.sum()), rtol=0, atol=LSE_ATOL,
                                           err_msg=f"{name} t={t} h={h} lse")
    assert_parity(np.stack(got_all), np.stack(ref_all), f"{name} sampled rows")

    print(f"[max] {name}: counts", flush=True)
    run(_zero_scale(g4, c))
    expect = _expected_counts(total, c.window, [p0, p0 + 1, total - 1])[p0:total]
    exact = expect <= EXACT_COUNT
    got = _counts(lse)
    rel = np.abs(np.exp(lse[0].cpu().numpy().astype(np.float64)) / expect[None, :] - 1.0)
    for h in range(c.Hq):
        np.testing.assert_array_equal(got[0, h][exact], expect[exact], err_msg=f"{name} counts h={h}")
    assert np.all(rel[:, ~exact] <= 4 * 2.0 ** -23 * 12.5), f"{name} counts past 2^17: {rel[:, ~exact].max()}"


def test_kv_decode_256k_sampled_heads_and_counts(gpu_lib):
    g4 = gpu_lib
    c = MAX_CONTEXT["31b_global_kv_decode_256k"]
    print("[256k] decode: inputs and run", flush=True)
    s = bench.build_decode(torch, g4, gen, c)
    assert int(s["n"].min()) == 262144 and int(s["max_len"]) == 262144
    lse = torch.empty((c.B, c.Hq), dtype=torch.float32, device="cuda")
    bench.run_decode_pro(g4, s)
    g4.g4attn_decode(s["desc"], s["q"].view(c.B, c.Hq, c.D), s["cache"], s["vcache"], s["kv_len"], s["max_len"],
                     s["out"], lse=lse, workspace=s["ws"])
    torch.cuda.synchronize()
    G = c.Hq // c.Hkv
    heads = [0, 7, 8, 31]
    got, ref = [], []
    for b in range(c.B):
        q = onr.norm_rope(f64(s["q_raw"][b:b + 1]), f64(s["wq"]), np.array([[int(s["L"][b])]]), c.rotary_dims,
                          c.theta)
        held = {}
        for h in heads:
            g = h // G
            if g not in held:
                held = {g: f64(s["cache"][b, g, :int(s["rows"][b])])}
            kk = held[g]
            sc = c.scale * (kk @ q[0, 0, h])
            m = sc.max()
            e = np.exp(sc - m)
            ref.append((e @ kk) / e.sum())
            got.append(f64(s["out"][b, h]))
            np.testing.assert_allclose(float(lse[b, h]), m + np.log(e.sum()), rtol=0, atol=LSE_ATOL,
                                       err_msg=f"256k decode b={b} h={h} lse")
    assert_parity(np.stack(got), np.stack(ref), "256k K=V decode sampled heads")

    desc0 = g4.layer_desc(c.Hq, c.Hkv, c.D, rotary_dims=c.rotary_dims, rope_theta=c.theta, scale=0.0)
    for splits in (0, 1, 8):          # 32, 1 and 8 chunks of 2^13, 2^18 and 2^15 rows
        print(f"[256k] decode counts, splits={splits}", flush=True)
        g4.g4attn_decode(desc0, s["q"].view(c.B, c.Hq, c.D), s["cache"], s["vcache"], s["kv_len"], s["max_len"],
                         s["out"], lse=lse, num_splits=splits)
        torch.cuda.synchronize()
        got_n = _counts(lse)
        for b in range(c.B):
            np.testing.assert_array_equal(got_n[b], np.full(c.Hq, int(s["n"][b])),
                                          err_msg=f"256k decode counts b={b} splits={splits}")
