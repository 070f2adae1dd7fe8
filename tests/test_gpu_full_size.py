"""Parity at the full workload sizes, in the launch configuration bench.py times.

Each test builds one workload with the bench's own builders (same seeded
generators, shapes and buffers), runs the whole hot path the way the bench
does (prologue kernels + attention), and compares sampled outputs with the
fp64 oracle computed one row (or one decode head) at a time from the raw
bf16 inputs.  The sampled rows cover the first and last tokens, tile and
window edges and seeded random positions in every KV group.
"""

import numpy as np
import pytest
import torch

import bench
from g4inputs import WORKLOADS, gen
from oracle import norm_rope as onr

from tests._cmp import assert_parity
from tests._rows import LSE_ATOL, prefill_oracle_rows, sample_tokens

pytestmark = pytest.mark.gpu

f64 = gen.to_f64

@pytest.mark.parametrize("name", ["e2b_sliding_prefill", "e2b_global_prefill", "31b_sliding_prefill",
                                  "31b_global_kv_prefill", "31b_sliding_image_prefill"])
def test_full_size_prefill_sampled_rows(gpu_lib, name):
    g4 = gpu_lib
    c = WORKLOADS[name]
    s = bench.build_prefill(torch, g4, gen, c)
    lse = torch.empty((c.B, c.Hq, c.S), dtype=torch.float32, device="cuda")
    bench.run_prefill(g4, s, lse=lse)
    torch.cuda.synchronize()
    G = c.Hq // c.Hkv
    got_all, ref_all = [], []
    for b in range(c.B):
        for g in range(c.Hkv):
            toks = sample_tokens(c.S, c.window, n_rand=6 if c.Hkv > 4 else 12, seed=(c.cfg_id, b, g))
            for st, n in c.images[:3]:      # rows at and inside image blocks
                toks = np.union1d(toks, [st, st + n // 2, st + n - 1])
            # two query heads of the group: the first and the last
            heads = sorted({g * G, g * G + G - 1})
            ro, rl = prefill_oracle_rows(s, b, g, toks, heads)
            ti = torch.as_tensor(toks, device="cuda")
            hi = torch.as_tensor(heads, device="cuda")
            got = f64(s["out"][b].index_select(0, ti).index_select(1, hi))
            got_lse = lse[b].index_select(0, hi).index_select(1, ti).T.cpu().numpy()
            np.testing.assert_allclose(got_lse, rl, rtol=0, atol=LSE_ATOL,
                                       err_msg=f"{name} b={b} g={g} lse")
            got_all.append(got)
            ref_all.append(ro)
    assert_parity(np.concatenate([x.reshape(-1) for x in got_all]),
                  np.concatenate([x.reshape(-1) for x in ref_all]), f"{name} sampled rows")


@pytest.mark.parametrize("name", ["31b_global_kv_decode", "31b_sliding_decode"])
def test_full_size_decode_sampled_heads(gpu_lib, name):
    g4 = gpu_lib
    c = WORKLOADS[name]
    s = bench.build_decode(torch, g4, gen, c)
    lse = torch.empty((c.B, c.Hq), dtype=torch.float32, device="cuda")
    bench.run_decode_pro(g4, s)
    g4.g4attn_decode(s["desc"], s["q"].view(c.B, c.Hq, c.D), s["cache"], s["vcache"], s["kv_len"], s["max_len"],
                     s["out"], lse=lse, workspace=s["ws"])
    torch.cuda.synchronize()
    L, n, rows = s["L"], s["n"], s["rows"]
    # the shortest and the longest sequence plus two seeded others; 8 heads each.
    # A sliding layer's ring holds min(n, window) rows, all visible to the new token.
    order = np.argsort(n)
    rng = np.random.default_rng(55)
    batch = sorted({int(order[0]), int(order[-1])} | set(rng.choice(c.B, size=2, replace=False).tolist()))
    heads = [0, 3, 4, 7, 8, 15, 16, 31] if c.Hkv == 4 else [0, 1, 2, 13, 16, 17, 30, 31]
    G = c.Hq // c.Hkv
    got, ref = [], []
    for b in batch:
        q = onr.norm_rope(f64(s["q_raw"][b:b + 1]), f64(s["wq"]), np.array([[L[b]]]), c.rotary_dims, c.theta)
        held = {}
        for h in heads:
            g = h // G
            if g not in held:                                   # one group's rows at a time
                kk = f64(s["cache"][b, g, :int(rows[b])])
                held = {g: (kk, kk if c.k_eq_v else f64(s["vcache"][b, g, :int(rows[b])]))}
            kk, vv = held[g]
            sc = c.scale * (kk @ q[0, 0, h])
            m = sc.max()
            e = np.exp(sc - m)
            ref.append((e @ vv) / e.sum())
            got.append(f64(s["out"][b, h]))
            np.testing.assert_allclose(float(lse[b, h]), m + np.log(e.sum()), rtol=0, atol=LSE_ATOL,
                                       err_msg=f"decode b={b} h={h} lse")
    assert_parity(np.stack(got), np.stack(ref), f"{name} sampled heads")


def test_full_size_chunk_prefill_sampled_rows(gpu_lib):
    """The 31B sliding chunked prefill (last 4096 of 16384 positions over linear caches), as timed."""
    g4 = gpu_lib
    c = WORKLOADS["31b_sliding_chunk_prefill"]
    s = bench.build_chunk(torch, g4, gen, c)
    lse = torch.empty((c.B, c.Hq, c.S), dtype=torch.float32, device="cuda")
    bench.run_chunk_pro(g4, s)
    g4.g4attn_prefill_chunk(s["desc"], s["q"], s["kc"], s["vc"], s["out"], s["pos0"], s["qlen"], s["total"] - 1,
                            lse=lse, workspace=s["ws"])
    torch.cuda.synchronize()
    G = c.Hq // c.Hkv
    got_all, ref_all = [], []
    for b in range(c.B):
        for g in (0, 7, 15):
            toks = sample_tokens(c.S, 0, n_rand=6, seed=(c.cfg_id, b, g))
            heads = [g * G, g * G + G - 1]
            for t in toks:
                p = s["p0"] + int(t)
                qraw = f64(s["q_raw"][b:b + 1, t:t + 1, heads])
                q = onr.norm_rope(qraw, f64(s["wq"]), np.array([[p]]), c.rotary_dims, c.theta)
                kk = f64(s["kc"][b, g, p - c.window + 1:p + 1])
                vv = f64(s["vc"][b, g, p - c.window + 1:p + 1])
                for hi_, h in enumerate(heads):
                    sc = c.scale * (kk @ q[0, 0, hi_])
                    m = sc.max()
                    e = np.exp(sc - m)
                    ref_all.append((e @ vv) / e.sum())
                    got_all.append(f64(s["out"][b, t, h]))
                    np.testing.assert_allclose(float(lse[b, h, t]), m + np.log(e.sum()), rtol=0, atol=LSE_ATOL)
    assert_parity(np.stack(got_all), np.stack(ref_all), "31b sliding chunk prefill sampled rows")


def test_full_size_kv_chunk_prefill_sampled_rows(gpu_lib):
    """The 31B K=V chunked prefill (last 4096 of 32768 positions over the raw-projection cache), as timed."""
    g4 = gpu_lib
    c = WORKLOADS["31b_global_kv_chunk_prefill"]
    s = bench.build_kv_chunk(torch, g4, gen, c)
    lse = torch.empty((c.B, c.Hq, c.S), dtype=torch.float32, device="cuda")
    bench.run_chunk_pro(g4, s)
    g4.g4attn_prefill_chunk_tied(s["desc"], s["q"], s["xc"], s["rc"], s["krc"], s["wk"], s["out"], s["pos0"],
                                 s["qlen"], s["total"] - 1, lse=lse, workspace=s["ws"])
    torch.cuda.synchronize()
    G = c.Hq // c.Hkv
    # the oracle's keys and values from the raw rows the cache was built from (same seeded draw)
    X = gen.normal_bf16((c.B, s["total"], c.Hkv, c.D), gen.seed_key(c.cfg_id, gen.X), "cuda")
    got_all, ref_all = [], []
    for g in (0, c.Hkv - 1):
        K, V = onr.kv_tied_k_v(f64(X[0:1, :, g:g + 1]), f64(s["wk"]), np.arange(s["total"])[None, :],
                               c.rotary_dims, c.theta)
        kk, vv = K[0, :, 0], V[0, :, 0]
        toks = sample_tokens(c.S, 0, n_rand=6, seed=(c.cfg_id, 0, g))
        heads = [g * G, g * G + G - 1]
        for t in toks:
            p = s["p0"] + int(t)
            qraw = f64(s["q_raw"][0:1, t:t + 1, heads])
            q = onr.norm_rope(qraw, f64(s["wq"]), np.array([[p]]), c.rotary_dims, c.theta)
            for hi_, h in enumerate(heads):
                sc = c.scale * (kk[:p + 1] @ q[0, 0, hi_])
                m = sc.max()
                e = np.exp(sc - m)
                ref_all.append((e @ vv[:p + 1]) / e.sum())
                got_all.append(f64(s["out"][0, t, h]))
                np.testing.assert_allclose(float(lse[0, h, t]), m + np.log(e.sum()), rtol=0, atol=LSE_ATOL)
    assert_parity(np.stack(got_all), np.stack(ref_all), "31B K=V chunk prefill sampled rows")


def test_full_size_raw_kv_decode_sampled_heads(gpu_lib):
    """The 31B K=V decode over the raw-projection cache (X + r + Krot), as timed."""
    g4 = gpu_lib
    c = WORKLOADS["31b_global_kv_decode_raw"]
    s = bench.build_decode_raw(torch, g4, gen, c)
    lse = torch.empty((c.B, c.Hq), dtype=torch.float32, device="cuda")
    bench.run_decode_pro(g4, s)
    g4.g4attn_decode_tied(s["desc"], s["q"].view(c.B, c.Hq, c.D), s["xc"], s["rc"], s["krc"], s["wk"], s["kv_len"],
                          s["max_len"], s["out"], lse=lse, workspace=s["ws"])
    torch.cuda.synchronize()
    L, n = s["L"], s["n"]
    order = np.argsort(n)
    batch = sorted({int(order[0]), int(order[-1]), 7})
    heads = [0, 7, 8, 31]
    G = c.Hq // c.Hkv
    got, ref = [], []
    for b in batch:
        q = onr.norm_rope(f64(s["q_raw"][b:b + 1]), f64(s["wq"]), np.array([[L[b]]]), c.rotary_dims, c.theta)
        for g in sorted({h // G for h in heads}):
            X = f64(s["xc"][b, g, :int(n[b])])[None, :, None, :]          # [1, n, 1, D] raw rows
            K, V = onr.kv_tied_k_v(X, f64(s["wk"]), np.arange(int(n[b]))[None, :], c.rotary_dims, c.theta)
            kk, vv = K[0, :, 0], V[0, :, 0]
            for h in [h for h in heads if h // G == g]:
                sc = c.scale * (kk @ q[0, 0, h])
                m = sc.max()
                e = np.exp(sc - m)
                ref.append((e @ vv) / e.sum())
                got.append(f64(s["out"][b, h]))
                np.testing.assert_allclose(float(lse[b, h]), m + np.log(e.sum()), rtol=0, atol=LSE_ATOL)
    assert_parity(np.stack(got), np.stack(ref), "31B raw K=V decode sampled heads")
