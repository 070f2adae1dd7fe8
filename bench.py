#!/usr/bin/env python3
"""Benchmark of the Gemma 4 31B attention hot path on one MI355X.

One step = one pass of every hot-path stage over the 31B-shaped workloads,
inputs resident in HBM:

  sliding prefill   B=2, S=16384, 32 q / 16 KV heads, D=256, window 1024:
                    q/k/v prologue (RMSNorm + RoPE) + attention
  global prefill    B=1, S=32768, 32 q / 4 KV heads, D=512, K=V tied:
                    q prologue + attention (K=V pre-pass included)
  global decode     B=32, one token each, KV lengths ~ U[32768, 131072],
                    32 q / 4 KV heads, D=512, one cache tensor for K and V:
                    q prologue at position = cache length + split-KV decode

and, reported beside them, the E2B sliding (B=1, S=1024, 8 q / 1 KV head,
D=256, window 512) and E2B global (B=1, S=8192, 8 q / 1 KV head, D=512,
separate K and V) prefills, the 31B sliding decode over rolling caches, the
31B sliding and K=V chunked prefills over caches, the image-span prefill and
the K=V decode over the raw-projection cache.

Prints one JSON line.  ``value`` is the prefill attention throughput
(algorithmic flops = 4*D per visible (row, key) pair per query head, over
both prefill calls); the decode stream rate, per-stage timings (median over
the timed steps, which every rate uses, and min), the roofline of the
dominant kernel and the CPU oracle baseline are in the same line.
"""

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E

# HBM bytes per launch of the K=V prefill main kernel from two rocprofv3
# counter runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch), each scaled by what
# the counter reads for a plain 1 GiB copy (x2.00 fetch, x1.00 write).  Valid
# only for the kernel sources they were taken on (hash below): once those
# change, the roofline reports traffic as null until the counters are re-taken.
PREFILL_TRAFFIC = {
    "sources": ["prefill.hip", "g4attn_internal.h", "norm_rope.hip", "abi.hip"],
    "sources_sha256": "dafcd3beb9b2e2e28e5634e334f40b9f4126815df21d7066560dad7991deaf3a",
    "fetch_kib": 3.23950e6, "fetch_scale": 2.0,
    "write_kib": 1.31073e6, "write_scale": 1.0,
}


# MFMA counters of the prefill main kernels from one rocprofv3 pass each
# (SQ_INSTS_VALU_MFMA_MOPS_BF16, SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE; per
# dispatch): counted flop = 512 x MOPS, busy = busy cycles / (1024 SIMDs x
# GRBM_GUI_ACTIVE / 8), average clock = (GRBM_GUI_ACTIVE / 8) / duration.
# The same source hash guards them.
PREFILL_MFMA = {
    "global": {"kernel": "prefill_kernel<512,K=V>", "counted_flop": 3.5219e13, "busy": 0.710,
               "avg_clock_GHz": 1.62, "duration_ms_under_counters": 29.24},
    "sliding": {"kernel": "prefill_d256_kernel", "counted_flop": 1.0984e12, "busy": 0.522,
                "avg_clock_GHz": 1.87, "duration_ms_under_counters": 1.077},
}


def sources_unchanged():
    """True while the kernel sources hash to the one the counters were taken on."""
    import hashlib
    csrc = os.path.join(ROOT, "decoder_attention_g4attn_amd", "csrc")
    h = hashlib.sha256()
    for f in PREFILL_TRAFFIC["sources"]:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest() == PREFILL_TRAFFIC["sources_sha256"]


def measured_traffic():
    """Scaled HBM bytes per launch of the K=V prefill kernel, or None if its sources changed."""
    if not sources_unchanged():
        return None
    t = PREFILL_TRAFFIC
    return (t["fetch_kib"] * t["fetch_scale"] + t["write_kib"] * t["write_scale"]) * 1024.0


def measured_mfma():
    """Counted MFMA work, utilisation and clock of the prefill kernels, or None if their sources changed."""
    return PREFILL_MFMA if sources_unchanged() else None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["sliding", "global", "decode", "sdecode", "chunk", "image", "rdecode",
                                       "e2b_sliding", "e2b_global", "kvchunk"],
                    default=None,
                    help="time one stage only (profiling aid)")
    ap.add_argument("--attainable", action="store_true",
                    help="run only the attainable-rate measurements (roofline probes, copy, GEMM) and print them")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 1 GiB device-to-device copy 3 times (HBM-counter calibration)")
    return ap.parse_args()


def copy_calibration():
    """A plain copy of known size: 1 GiB read + 1 GiB written per launch."""
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read_per_launch": n, "copy_bytes_written_per_launch": n, "launches": 3}))


def attainable(torch):
    """Measured attainable rates on this GPU, as context for the roofline
    fractions: the two roofline probes of libg4probe.so (a bare bf16 MFMA
    loop, one workgroup of 4 waves per CU for ~30 ms like the K=V prefill,
    on random operands like the attention's data and again on operands that
    barely switch, which let the chip hold its clock; and an 8 GiB non-temporal
    streaming read), a plain device copy of 2 GiB
    (read + write bytes over time) and a large bf16 GEMM through torch (the
    vendor library's MFMA path)."""
    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps
    n = 2 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    ms = timed(lambda: dst.copy_(src), 5)
    copy_gbps = 2.0 * n / ms / 1e6
    del src, dst
    m = 8192
    a = torch.randn(m, m, device="cuda").to(torch.bfloat16)
    b = torch.randn(m, m, device="cuda").to(torch.bfloat16)
    ms = timed(lambda: torch.matmul(a, b), 5)
    gemm = 2.0 * m ** 3 / ms / 1e9
    del a, b
    from decoder_attention_g4attn_amd import probe
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(cus * 256, dtype=torch.float32, device="cuda")
    iters = 1 << 18
    flop = float(cus) * 4 * iters * 8 * 32768
    ms = timed(lambda: probe.mfma_bf16(out, cus, iters, probe.RANDOM), 3)
    mfma = flop / ms / 1e9
    ms = timed(lambda: probe.mfma_bf16(out, cus, iters, probe.LOW_ACTIVITY), 3)
    mfma_low = flop / ms / 1e9
    del out
    src = torch.empty(8 << 30, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    wgs = 2 * cus
    sink = torch.empty(wgs * 256, dtype=torch.int32, device="cuda")
    ms = timed(lambda: probe.stream_read(src, sink, wgs), 5)
    rd = float(src.numel()) / ms / 1e6
    del src, sink
    return {"mfma_loop_bf16_tflops": round(mfma, 1), "mfma_loop_bf16_low_activity_tflops": round(mfma_low, 1),
            "stream_read_GBps": round(rd, 1),
            "hbm_copy_GBps": round(copy_gbps, 1), "bf16_gemm_8192_tflops": round(gemm, 1)}


class Stage:
    def __init__(self, name):
        self.name = name
        self.ms = []


def build_prefill(torch, g4, gen, c):
    """Raw (pre-prologue) inputs and output buffers of one prefill workload."""
    dev = "cuda"
    q_raw = gen.normal_bf16((c.B, c.S, c.Hq, c.D), gen.seed_key(c.cfg_id, gen.Q), dev)
    wq = gen.norm_weight(c.D, gen.seed_key(c.cfg_id, gen.WQ)).to(dev)
    wk = gen.norm_weight(c.D, gen.seed_key(c.cfg_id, gen.WK)).to(dev)
    desc = g4.layer_desc(c.Hq, c.Hkv, c.D, window=c.window, k_eq_v=c.k_eq_v, rotary_dims=c.rotary_dims,
                         rope_theta=c.theta)
    s = dict(c=c, desc=desc, q_raw=q_raw, wq=wq, wk=wk, q=torch.empty_like(q_raw), out=torch.empty_like(q_raw),
             span_lo=None, span_hi=None)
    if c.images:
        lo, hi = gen.image_spans(c.S, c.images)
        s["span_lo"] = torch.from_numpy(np.tile(lo, (c.B, 1))).to(dev)
        s["span_hi"] = torch.from_numpy(np.tile(hi, (c.B, 1))).to(dev)
    if c.k_eq_v:
        s["X"] = gen.normal_bf16((c.B, c.S, c.Hkv, c.D), gen.seed_key(c.cfg_id, gen.X), dev)
        s["ws"] = torch.empty(g4.g4attn_prefill_workspace_bytes(desc, c.B, c.S), dtype=torch.uint8, device=dev)
    else:
        s["k_raw"] = gen.normal_bf16((c.B, c.S, c.Hkv, c.D), gen.seed_key(c.cfg_id, gen.K), dev)
        s["v_raw"] = gen.normal_bf16((c.B, c.S, c.Hkv, c.D), gen.seed_key(c.cfg_id, gen.V), dev)
        s["k"] = torch.empty_like(s["k_raw"])
        s["v"] = torch.empty_like(s["v_raw"])
        s["ws"] = torch.empty(g4.g4attn_prefill_workspace_bytes(desc, c.B, c.S), dtype=torch.uint8, device=dev)
    return s


def build_decode(torch, g4, gen, c):
    """KV cache(s) of post-prologue rows, raw queries and buffers of a decode workload.

    Global K=V layer: one cache [B, Hkv, cap, D] holds rows 0..L_b (the new
    token's own row is slot L_b).  Sliding layer: separate K and V rolling
    caches of `window` slots holding the last min(L_b + 1, window) positions
    (position p in slot p mod window; every slot once L_b + 1 >= window).
    """
    dev = "cuda"
    L = gen.decode_lengths(c.B, c.len_lo, c.len_hi, gen.seed_key(c.cfg_id, gen.LENS))
    n = L.astype(np.int64) + 1            # positions so far, the new token included
    cap = c.cache_cap
    rows = np.minimum(n, cap) if c.window else n
    caches = []
    for which in ((gen.CACHE,) if c.k_eq_v else (gen.CACHE, gen.CACHE_V)):
        cache = torch.empty((c.B, c.Hkv, cap, c.D), dtype=torch.bfloat16, device=dev)
        for b in range(c.B):
            cache[b, :, :rows[b]] = gen.normal_bf16((c.Hkv, int(rows[b]), c.D), gen.seed_key(c.cfg_id, which, b), dev)
        caches.append(cache)
    q_raw = gen.normal_bf16((c.B, 1, c.Hq, c.D), gen.seed_key(c.cfg_id, gen.QDEC), dev)
    wq = gen.norm_weight(c.D, gen.seed_key(c.cfg_id, gen.WQ)).to(dev)
    desc = g4.layer_desc(c.Hq, c.Hkv, c.D, window=c.window, rotary_dims=c.rotary_dims, rope_theta=c.theta)
    pos0 = torch.from_numpy(L.astype(np.int32)).to(dev)
    kv_len = torch.from_numpy(n.astype(np.int32)).to(dev)
    max_len = int(n.max())
    dws = torch.empty(g4.g4attn_decode_workspace_bytes(desc, c.B, max_len, 0), dtype=torch.uint8, device=dev)
    return dict(c=c, desc=desc, cache=caches[0], vcache=caches[-1], q_raw=q_raw, wq=wq, pos0=pos0,
                kv_len=kv_len, L=L, max_len=max_len, max_pos=int(L.max()), n=n, rows=rows,
                q=torch.empty((c.B, 1, c.Hq, c.D), dtype=torch.bfloat16, device=dev),
                out=torch.empty((c.B, c.Hq, c.D), dtype=torch.bfloat16, device=dev), ws=dws)


def build_decode_raw(torch, g4, gen, c):
    """K=V decode over the raw-projection cache: X rows 0..L_b of every sequence
    (drawn like the pre-normed cache) with their inverse RMS and rotated key
    part appended by g4attn_kv_tied_append (set-up, not timed)."""
    dev = "cuda"
    L = gen.decode_lengths(c.B, c.len_lo, c.len_hi, gen.seed_key(c.cfg_id, gen.LENS))
    n = L.astype(np.int64) + 1
    cap = c.cache_cap
    xc = torch.empty((c.B, c.Hkv, cap, c.D), dtype=torch.bfloat16, device=dev)
    for b in range(c.B):
        xc[b, :, :n[b]] = gen.normal_bf16((c.Hkv, int(n[b]), c.D), gen.seed_key(c.cfg_id, gen.CACHE, b), dev)
    rc = torch.empty((c.B, c.Hkv, cap), dtype=torch.float32, device=dev)
    krc = torch.empty((c.B, c.Hkv, cap, 128), dtype=torch.bfloat16, device=dev)
    wk = gen.norm_weight(c.D, gen.seed_key(c.cfg_id, gen.WK)).to(dev)
    for b in range(c.B):   # the cache's own X rows as the projection [1, n_b, Hkv, D] (strided view)
        xv = xc[b:b + 1, :, :n[b]].permute(0, 2, 1, 3)
        g4.g4attn_kv_tied_append(xv, wk, xc[b:b + 1], rc[b:b + 1], krc[b:b + 1], c.theta)
    q_raw = gen.normal_bf16((c.B, 1, c.Hq, c.D), gen.seed_key(c.cfg_id, gen.QDEC), dev)
    wq = gen.norm_weight(c.D, gen.seed_key(c.cfg_id, gen.WQ)).to(dev)
    desc = g4.layer_desc(c.Hq, c.Hkv, c.D, window=0, k_eq_v=True, rotary_dims=c.rotary_dims, rope_theta=c.theta)
    max_len = int(n.max())
    dws = torch.empty(g4.g4attn_decode_workspace_bytes(desc, c.B, max_len, 0), dtype=torch.uint8, device=dev)
    return dict(c=c, desc=desc, xc=xc, rc=rc, krc=krc, wk=wk, q_raw=q_raw, wq=wq, L=L, n=n,
                pos0=torch.from_numpy(L.astype(np.int32)).to(dev), kv_len=torch.from_numpy(n.astype(np.int32)).to(dev),
                max_len=max_len, max_pos=int(L.max()),
                q=torch.empty((c.B, 1, c.Hq, c.D), dtype=torch.bfloat16, device=dev),
                out=torch.empty((c.B, c.Hq, c.D), dtype=torch.bfloat16, device=dev), ws=dws)


def run_decode_raw_attn(g4, s):
    g4.g4attn_decode_tied(s["desc"], s["q"].view(s["q"].shape[0], s["q"].shape[2], s["q"].shape[3]), s["xc"],
                          s["rc"], s["krc"], s["wk"], s["kv_len"], s["max_len"], s["out"], workspace=s["ws"])


def build_chunk(torch, g4, gen, c):
    """Chunked prefill: the last c.S of c.len_hi positions of each sequence; linear K and V
    caches [B, Hkv, len_hi, D] hold every position (post-prologue rows), the chunk's included."""
    dev = "cuda"
    total = c.len_hi
    kc = gen.normal_bf16((c.B, c.Hkv, total, c.D), gen.seed_key(c.cfg_id, gen.CACHE), dev)
    vc = gen.normal_bf16((c.B, c.Hkv, total, c.D), gen.seed_key(c.cfg_id, gen.CACHE_V), dev)
    q_raw = gen.normal_bf16((c.B, c.S, c.Hq, c.D), gen.seed_key(c.cfg_id, gen.Q), dev)
    wq = gen.norm_weight(c.D, gen.seed_key(c.cfg_id, gen.WQ)).to(dev)
    desc = g4.layer_desc(c.Hq, c.Hkv, c.D, window=c.window, rotary_dims=c.rotary_dims, rope_theta=c.theta)
    p0 = total - c.S
    ws = torch.empty(g4.g4attn_prefill_workspace_bytes(desc, c.B, c.S), dtype=torch.uint8, device=dev)
    return dict(c=c, desc=desc, kc=kc, vc=vc, q_raw=q_raw, wq=wq, p0=p0, total=total,
                pos0=torch.full((c.B,), p0, dtype=torch.int32, device=dev),
                qlen=torch.full((c.B,), c.S, dtype=torch.int32, device=dev),
                q=torch.empty_like(q_raw), out=torch.empty_like(q_raw), ws=ws)


def build_kv_chunk(torch, g4, gen, c):
    """Chunked prefill of a K=V layer: the last c.S of c.len_hi positions over the layer's own
    cache (raw projection X, its inverse RMS and rotated key part; every position written by
    g4attn_kv_tied_append at set-up, not timed)."""
    dev = "cuda"
    total = c.len_hi
    X = gen.normal_bf16((c.B, total, c.Hkv, c.D), gen.seed_key(c.cfg_id, gen.X), dev)
    wk = gen.norm_weight(c.D, gen.seed_key(c.cfg_id, gen.WK)).to(dev)
    xc = torch.empty((c.B, c.Hkv, total, c.D), dtype=torch.bfloat16, device=dev)
    rc = torch.empty((c.B, c.Hkv, total), dtype=torch.float32, device=dev)
    krc = torch.empty((c.B, c.Hkv, total, 128), dtype=torch.bfloat16, device=dev)
    g4.g4attn_kv_tied_append(X, wk, xc, rc, krc, c.theta)
    del X
    q_raw = gen.normal_bf16((c.B, c.S, c.Hq, c.D), gen.seed_key(c.cfg_id, gen.Q), dev)
    wq = gen.norm_weight(c.D, gen.seed_key(c.cfg_id, gen.WQ)).to(dev)
    desc = g4.layer_desc(c.Hq, c.Hkv, c.D, window=c.window, k_eq_v=True, rotary_dims=c.rotary_dims,
                         rope_theta=c.theta)
    p0 = total - c.S
    ws = torch.empty(g4.g4attn_prefill_workspace_bytes(desc, c.B, c.S), dtype=torch.uint8, device=dev)
    return dict(c=c, desc=desc, xc=xc, rc=rc, krc=krc, wk=wk, q_raw=q_raw, wq=wq, p0=p0, total=total,
                pos0=torch.full((c.B,), p0, dtype=torch.int32, device=dev),
                qlen=torch.full((c.B,), c.S, dtype=torch.int32, device=dev),
                q=torch.empty_like(q_raw), out=torch.empty_like(q_raw), ws=ws)


def build_workloads(torch, g4, gen, W, keys=None):
    """Inputs of every stage's workload (or of ``keys`` only)."""
    builders = {"e2b_sliding": (build_prefill, "e2b_sliding_prefill"),
                "e2b_global": (build_prefill, "e2b_global_prefill"),
                "kvchunk": (build_kv_chunk, "31b_global_kv_chunk_prefill"),
                "sliding": (build_prefill, "31b_sliding_prefill"),
                "global": (build_prefill, "31b_global_kv_prefill"),
                "decode": (build_decode, "31b_global_kv_decode"),
                "sdecode": (build_decode, "31b_sliding_decode"),
                "chunk": (build_chunk, "31b_sliding_chunk_prefill"),
                "image": (build_prefill, "31b_sliding_image_prefill"),
                "rdecode": (build_decode_raw, "31b_global_kv_decode_raw")}
    st = {k: fn(torch, g4, gen, W[name]) for k, (fn, name) in builders.items() if keys is None or k in keys}
    torch.cuda.synchronize()
    return st


def run_sliding(g4, s):
    c = s["c"]
    g4.g4attn_norm_rope(s["q_raw"], s["q"], s["wq"], c.D, c.rotary_dims, c.theta)
    g4.g4attn_norm_rope(s["k_raw"], s["k"], s["wk"], c.D, c.rotary_dims, c.theta)
    g4.g4attn_norm_rope(s["v_raw"], s["v"], None, c.D, 0, c.theta)


def run_sliding_attn(g4, s):
    g4.g4attn_prefill(s["desc"], s["q"], s["k"], s["v"], s["out"], workspace=s["ws"])


def run_prefill(g4, s, lse=None):
    """The whole prefill hot path of one workload: prologue(s) + attention."""
    c = s["c"]
    g4.g4attn_norm_rope(s["q_raw"], s["q"], s["wq"], c.D, c.rotary_dims, c.theta)
    if c.k_eq_v:
        g4.g4attn_prefill(s["desc"], s["q"], s["X"], None, s["out"], w_k=s["wk"], lse=lse, workspace=s["ws"])
    else:
        g4.g4attn_norm_rope(s["k_raw"], s["k"], s["wk"], c.D, c.rotary_dims, c.theta)
        g4.g4attn_norm_rope(s["v_raw"], s["v"], None, c.D, 0, c.theta)
        g4.g4attn_prefill(s["desc"], s["q"], s["k"], s["v"], s["out"], lse=lse, workspace=s["ws"],
                          span_lo=s["span_lo"], span_hi=s["span_hi"])


def run_global_pro(g4, s):
    c = s["c"]
    g4.g4attn_norm_rope(s["q_raw"], s["q"], s["wq"], c.D, c.rotary_dims, c.theta)


def run_global_attn(g4, s):
    g4.g4attn_prefill(s["desc"], s["q"], s["X"], None, s["out"], w_k=s["wk"], workspace=s["ws"])


def run_decode_pro(g4, s):
    c = s["c"]
    g4.g4attn_norm_rope(s["q_raw"], s["q"], s["wq"], c.D, c.rotary_dims, c.theta, pos0=s["pos0"],
                        max_pos=s["max_pos"])


def run_image_attn(g4, s):
    g4.g4attn_prefill(s["desc"], s["q"], s["k"], s["v"], s["out"], workspace=s["ws"], span_lo=s["span_lo"],
                      span_hi=s["span_hi"])


def visible_pairs(S, window):
    """Visible (row, key) pairs of one head: row i sees min(i+1, w) keys (all i+1 if global)."""
    if window == 0 or S <= window:
        return S * (S + 1) // 2
    return window * (window + 1) // 2 + (S - window) * window


def span_pairs(S, window, lo, hi):
    """Visible (row, key) pairs of one head with bidirectional spans [lo, hi]:
    the window's (or causal) keys plus each row's span keys outside them."""
    i = np.arange(S, dtype=np.int64)
    lo, hi = np.asarray(lo, np.int64), np.asarray(hi, np.int64)
    base = np.minimum(i + 1, window) if window else i + 1
    first = i - window + 1 if window else np.zeros_like(i)     # lowest key of the window
    return int((base + (hi - i) + np.maximum(0, first - lo)).sum())


def run_chunk_pro(g4, s):
    c = s["c"]
    g4.g4attn_norm_rope(s["q_raw"], s["q"], s["wq"], c.D, c.rotary_dims, c.theta, pos0=s["pos0"],
                        max_pos=s["total"] - 1)


def run_chunk_attn(g4, s):
    g4.g4attn_prefill_chunk(s["desc"], s["q"], s["kc"], s["vc"], s["out"], s["pos0"], s["qlen"], s["total"] - 1,
                            workspace=s["ws"])


def run_kv_chunk_attn(g4, s):
    g4.g4attn_prefill_chunk_tied(s["desc"], s["q"], s["xc"], s["rc"], s["krc"], s["wk"], s["out"], s["pos0"],
                                 s["qlen"], s["total"] - 1, workspace=s["ws"])


def run_decode_attn(g4, s):
    g4.g4attn_decode(s["desc"], s["q"].view(s["q"].shape[0], s["q"].shape[2], s["q"].shape[3]),
                     s["cache"], s["vcache"], s["kv_len"], s["max_len"], s["out"], workspace=s["ws"])


def cpu_info():
    """Host cores this process may run on, the BLAS thread count and the CPU model."""
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        blas = None
    model = None
    try:
        import subprocess
        txt = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=20).stdout
        for line in txt.splitlines():
            if line.startswith("Model name:"):
                model = line.split(":", 1)[1].strip()
                break
    except Exception:
        pass
    return cores, blas, model


def cpu_baseline(torch, gen, st, log, budget_s=10.0):
    """The fp64 oracle, timed on the host cores, per config, from the same raw
    (pre-prologue) seeded inputs as the GPU: prologue (RMSNorm + RoPE) and
    attention are both inside the timed region; the rates count the same
    algorithmic attention flops (4*D per visible pair per query head) or
    cache bytes as the GPU's.

    E2B sliding, E2B global and 31B sliding prefill and the 31B K=V decode
    run in full.  The 31B K=V global prefill (35 TFLOP, hours in fp64) runs on
    a row sample: KV group 0, its 8 query heads, the last R rows, each seeing
    every earlier key; R doubled until the run takes about budget_s / 3.  The headline value is the oracle's rate
    over the two 31B prefill calls (31B sliding in full + the K=V sample),
    the same quantity as the GPU's value.
    """
    from oracle import attention as oat
    from oracle import norm_rope as onr
    f64 = gen.to_f64
    torch.cuda.synchronize()
    per = {}

    def prefill_full(key):
        s = st[key]
        c = s["c"]
        qr, kr, vr = f64(s["q_raw"]), f64(s["k_raw"]), f64(s["v_raw"])
        wq, wk = f64(s["wq"]), f64(s["wk"])
        pos = np.tile(np.arange(c.S), (c.B, 1))
        t0 = time.perf_counter()
        q = onr.norm_rope(qr, wq, pos, c.rotary_dims, c.theta)
        k = onr.norm_rope(kr, wk, pos, c.rotary_dims, c.theta)
        v = onr.norm_rope(vr, None, pos, 0, c.theta)
        oat.attention_band(q, k, v, c.scale, c.window)
        dt = time.perf_counter() - t0
        fl = 4.0 * c.D * visible_pairs(c.S, c.window) * c.Hq * c.B
        per[c.name] = {"value": round(fl / dt / 1e12, 5), "unit": "TFLOP/s", "seconds": round(dt, 2),
                       "sample": "full (prologue + attention)"}
        return fl, dt

    for key in ("e2b_sliding", "e2b_global", "sliding"):
        log(f"oracle: {st[key]['c'].name} in full")
        fl, dt = prefill_full(key)
        if key == "sliding":
            fl_s, dt_s = fl, dt

    # 31B K=V global prefill: KV group 0, last R rows
    log("oracle: 31b_global_kv_prefill row sample")
    s = st["global"]
    c = s["c"]
    G = c.Hq // c.Hkv
    S = c.S
    X = f64(s["X"][0:1, :, 0:1])                      # [1, S, 1, D] raw tied projection, group 0
    wk, wq = f64(s["wk"]), f64(s["wq"])
    R = 16
    while True:
        rows = np.arange(S - R, S)
        qr = f64(s["q_raw"][0:1, S - R:, :G])          # [1, R, G, D]
        t0 = time.perf_counter()
        K, V = onr.kv_tied_k_v(X, wk, np.arange(S)[None, :], c.rotary_dims, c.theta)
        q = onr.norm_rope(qr, wq, rows[None, :], c.rotary_dims, c.theta)
        qfull = np.zeros((1, S, G, c.D))
        qfull[0, S - R:] = q[0]
        oat.attention_band(qfull, K, V, c.scale, 0, rows=rows)
        dt = time.perf_counter() - t0
        pairs = int((rows + 1).sum()) * G
        if dt > budget_s / 3 or R >= min(4096, S):
            break
        R = min(2 * R, S)
    fl_g = 4.0 * c.D * pairs
    per[c.name] = {"value": round(fl_g / dt / 1e12, 5), "unit": "TFLOP/s", "seconds": round(dt, 2),
                   "sample": f"KV group 0 ({G} q heads), last {R} rows x all earlier keys ({pairs} visible "
                             f"pairs of {visible_pairs(S, 0) * c.Hq}); K/V prologue of the group's {S} rows "
                             f"and the rows' q prologue included"}

    # 31B K=V decode: every sequence (the cache slice of one sequence is widened to fp64 at a time)
    log("oracle: 31b_global_kv_decode in full")
    s = st["decode"]
    c = s["c"]
    nseq = c.B
    t_dec, nbytes = 0.0, 0.0
    for b in range(nseq):
        nb = int(s["n"][b])
        kc = f64(s["cache"][b:b + 1, :, :nb])          # [1, Hkv, n_b, D]
        qr = f64(s["q_raw"][b:b + 1])                  # [1, 1, Hq, D]
        t0 = time.perf_counter()
        q = onr.norm_rope(qr, f64(s["wq"]), np.array([[int(s["L"][b])]]), c.rotary_dims, c.theta)
        oat.decode_attention(q[:, 0], kc, kc, np.array([nb]), c.scale)
        t_dec += time.perf_counter() - t0
        nbytes += float(nb) * c.Hkv * c.D * 2 + 2.0 * c.Hq * c.D * 2
        del kc
    per[c.name] = {"value": round(nbytes / t_dec / 1e9, 4), "unit": "GB/s", "seconds": round(t_dec, 2),
                   "sample": f"full: all {nseq} sequences ({int(s['n'].sum())} cached rows), every head, "
                             f"q prologue included (the fp64 widening of each cache slice is not timed)"}

    cores, blas, model = cpu_info()
    value = (fl_s + fl_g) / (dt_s + dt) / 1e12
    return {"value": round(value, 5), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": "31B sliding prefill in full + 31B K=V global prefill row sample "
                      f"({per['31b_global_kv_prefill']['sample']}); fp64 numpy, prologue + attention timed",
            "blas_threads": blas, "cpu_model": model, "per_config": per}


def _r(res, key, nd):
    return round(res[key], nd) if key in res else None


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.attainable:
        import torch
        print(json.dumps(attainable(torch)))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the attention path shards by KV head / batch without collectives).", file=sys.stderr)
        sys.exit(2)
    import torch
    import decoder_attention_g4attn_amd as g4
    from g4inputs import WORKLOADS, gen

    g4.load()
    torch.cuda.set_device(0)
    log = lambda m: print(f"[bench] {m}", file=sys.stderr, flush=True)
    log("generating inputs")
    st = build_workloads(torch, g4, gen, WORKLOADS, keys=[args.only] if args.only else None)
    log("inputs ready")

    plan = [("e2b_sliding_prologue", run_sliding, "e2b_sliding"), ("e2b_sliding_attn", run_sliding_attn, "e2b_sliding"),
            ("e2b_global_prologue", run_sliding, "e2b_global"), ("e2b_global_attn", run_sliding_attn, "e2b_global"),
            ("sliding_prologue", run_sliding, "sliding"), ("sliding_attn", run_sliding_attn, "sliding"),
            ("global_prologue", run_global_pro, "global"), ("global_attn", run_global_attn, "global"),
            ("decode_prologue", run_decode_pro, "decode"), ("decode_attn", run_decode_attn, "decode"),
            ("sliding_decode_prologue", run_decode_pro, "sdecode"),
            ("sliding_decode_attn", run_decode_attn, "sdecode"),
            ("chunk_prologue", run_chunk_pro, "chunk"), ("chunk_attn", run_chunk_attn, "chunk"),
            ("image_prologue", run_sliding, "image"), ("image_attn", run_image_attn, "image"),
            ("raw_decode_prologue", run_decode_pro, "rdecode"), ("raw_decode_attn", run_decode_raw_attn, "rdecode"),
            ("kv_chunk_prologue", run_chunk_pro, "kvchunk"), ("kv_chunk_attn", run_kv_chunk_attn, "kvchunk")]
    if args.only:
        plan = [p for p in plan if p[2] == args.only]

    def step(record):
        evs = []
        for name, fn, key in plan:
            if record:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                fn(g4, st[key])
                e1.record()
                evs.append((name, e0, e1))
            else:
                fn(g4, st[key])
        return evs

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")
    all_evs = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        all_evs.append(step(True))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log(f"timed {args.steps} steps in {wall:.2f}s")
    ms = {}
    for evs in all_evs:
        for name, e0, e1 in evs:
            ms.setdefault(name, []).append(e0.elapsed_time(e1))
    # per-stage median over the timed steps drives every rate; min is reported beside it
    avg = {k: float(np.median(v)) for k, v in ms.items()}
    mins = {k: float(np.min(v)) for k, v in ms.items()}

    W = WORKLOADS
    cs, cg = W["31b_sliding_prefill"], W["31b_global_kv_prefill"]
    fl_sliding = 4.0 * cs.D * visible_pairs(cs.S, cs.window) * cs.Hq * cs.B
    fl_global = 4.0 * cg.D * visible_pairs(cg.S, 0) * cg.Hq * cg.B
    res = {}

    def prefill_rate(stage, key, flops):
        if stage in avg:
            res[key] = flops / avg[stage] / 1e9

    prefill_rate("sliding_attn", "sliding_prefill_tflops", fl_sliding)
    prefill_rate("global_attn", "global_prefill_tflops", fl_global)
    for key, name in (("e2b_sliding", "e2b_sliding_prefill"), ("e2b_global", "e2b_global_prefill")):
        ce = W[name]
        prefill_rate(key + "_attn", key + "_prefill_tflops",
                     4.0 * ce.D * visible_pairs(ce.S, ce.window) * ce.Hq * ce.B)
    cc = W["31b_sliding_chunk_prefill"]
    # chunk row p sees min(p + 1, window) keys
    prefill_rate("chunk_attn", "chunk_prefill_tflops",
                 4.0 * cc.D * sum(min(p + 1, cc.window) for p in range(cc.len_hi - cc.S, cc.len_hi)) * cc.Hq * cc.B)
    ck = W["31b_global_kv_chunk_prefill"]
    # K=V chunk row p sees every key 0..p
    prefill_rate("kv_chunk_attn", "kv_chunk_prefill_tflops",
                 4.0 * ck.D * sum(p + 1 for p in range(ck.len_hi - ck.S, ck.len_hi)) * ck.Hq * ck.B)
    ci = W["31b_sliding_image_prefill"]
    prefill_rate("image_attn", "image_prefill_tflops",
                 4.0 * ci.D * span_pairs(ci.S, ci.window, *gen.image_spans(ci.S, ci.images)) * ci.Hq * ci.B)
    if "decode_attn" in avg:
        cd, dec = W["31b_global_kv_decode"], st["decode"]
        # one cache tensor serves as K and V: D bf16 per row per KV head, plus q in and out
        dec_bytes = float(dec["n"].sum()) * cd.Hkv * cd.D * 2 + 2.0 * cd.B * cd.Hq * cd.D * 2
        res["decode_GBps"] = dec_bytes / avg["decode_attn"] / 1e6
    if "sliding_decode_attn" in avg:
        csd, sdec = W["31b_sliding_decode"], st["sdecode"]
        # separate K and V rings: 2 * D bytes per row per KV head for each
        sdec_bytes = float(sdec["rows"].sum()) * csd.Hkv * csd.D * 2 * 2 + 2.0 * csd.B * csd.Hq * csd.D * 2
        res["sliding_decode_GBps"] = sdec_bytes / avg["sliding_decode_attn"] / 1e6
    if "raw_decode_attn" in avg:
        crd, rd = W["31b_global_kv_decode_raw"], st["rdecode"]
        # X row (2 D bytes) + rotated key part (256 bytes) + inverse RMS (4 bytes) per row per KV head
        rdec_bytes = float(rd["n"].sum()) * crd.Hkv * (crd.D * 2 + 256 + 4) + 2.0 * crd.B * crd.Hq * crd.D * 2
        res["raw_kv_decode_GBps"] = rdec_bytes / avg["raw_decode_attn"] / 1e6
    # prologues (norm + RoPE): 2 bytes read and 2 written per element of q (and k, v)
    pro = {}
    for stage, name, tensors in (("sliding_prologue", "31b_sliding_prefill", "qkv"),
                                 ("global_prologue", "31b_global_kv_prefill", "q"),
                                 ("e2b_global_prologue", "e2b_global_prefill", "qkv")):
        if stage in avg:
            cw = W[name]
            elems = cw.B * cw.S * cw.D * (cw.Hq + (2 * cw.Hkv if tensors == "qkv" else 0))
            pro[stage] = round(4.0 * elems / avg[stage] / 1e6, 1)
    prefill_ms = avg.get("sliding_attn", 0.0) + avg.get("global_attn", 0.0)
    prefill_fl = (fl_sliding if "sliding_attn" in avg else 0) + (fl_global if "global_attn" in avg else 0)
    value = prefill_fl / prefill_ms / 1e9 if prefill_ms > 0 else None
    ms_per_step = wall * 1e3 / args.steps

    roof = None
    if "global_attn" in avg:
        ach = res["global_prefill_tflops"]
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic(),
                "traffic_unit": "bytes per launch (HBM, rocprofv3 FETCH_SIZE+WRITE_SIZE, copy-calibrated)",
                "kernel": "g4attn_prefill on the 31B K=V global layer (K=V pre-pass + prefill_kernel<512,K=V>)",
                "flops_per_launch": fl_global,
                "mfma_counters": measured_mfma()}
    out = {
        "metric": "prefill attention TFLOP/s (31B global/sliding) + decode KV GB/s, 1xMI355X",
        "value": round(value, 3) if value else None,
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {
            "workload": "Gemma 4 31B attention layers: sliding prefill B2 S16384 Hq32 Hkv16 D256 w1024; "
                        "global K=V prefill B1 S32768 Hq32 Hkv4 D512; global K=V decode B32 "
                        "L~U[32768,131072] Hq32 Hkv4 D512",
            "value_is": "prefill attention TFLOP/s over the two 31B prefill calls",
            "parallelism": "single GPU",
        },
        "decode_GBps": _r(res, "decode_GBps", 1),
        "decode_hbm_frac": round(res["decode_GBps"] / PEAK_HBM_GBPS, 4) if "decode_GBps" in res else None,
        "sliding_decode_GBps": _r(res, "sliding_decode_GBps", 1),
        "chunk_prefill_tflops": _r(res, "chunk_prefill_tflops", 2),
        "image_prefill_tflops": _r(res, "image_prefill_tflops", 2),
        "raw_kv_decode_GBps": _r(res, "raw_kv_decode_GBps", 1),
        "sliding_prefill_tflops": _r(res, "sliding_prefill_tflops", 2),
        "global_prefill_tflops": _r(res, "global_prefill_tflops", 2),
        "e2b_sliding_prefill_tflops": _r(res, "e2b_sliding_prefill_tflops", 2),
        "e2b_global_prefill_tflops": _r(res, "e2b_global_prefill_tflops", 2),
        "kv_chunk_prefill_tflops": _r(res, "kv_chunk_prefill_tflops", 2),
        # every prefill rate as a fraction of the bf16 dense MFMA peak, every decode rate of HBM peak
        "prologue_GBps": pro,
        "frac_of_peak": {k: round(v / (PEAK_HBM_GBPS if k.endswith("GBps") else PEAK_BF16_TFLOPS), 4)
                         for k, v in sorted(res.items())},
        "stage_ms": {k: round(v, 4) for k, v in avg.items()},
        "stage_ms_min": {k: round(v, 4) for k, v in mins.items()},
        "roofline": roof,
    }
    if args.only is None:
        log("measuring attainable rates: MFMA loop, streaming read, copy, GEMM")
        att = attainable(torch)
        att["global_prefill_frac_of_mfma_loop"] = round(res["global_prefill_tflops"] / att["mfma_loop_bf16_tflops"], 4)
        att["sliding_prefill_frac_of_mfma_loop"] = round(res["sliding_prefill_tflops"] / att["mfma_loop_bf16_tflops"],
                                                         4)
        att["decode_frac_of_stream_read"] = round(res["decode_GBps"] / att["stream_read_GBps"], 4)
        att["global_prefill_frac_of_gemm"] = round(res["global_prefill_tflops"] / att["bf16_gemm_8192_tflops"], 4)
        att["decode_frac_of_copy"] = round(res["decode_GBps"] / att["hbm_copy_GBps"], 4)
        out["attainable"] = att
    if not args.no_cpu_baseline and args.only is None:
        log("timing the CPU oracle on a sample")
        out["cpu_baseline"] = cpu_baseline(torch, gen, st, log)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
