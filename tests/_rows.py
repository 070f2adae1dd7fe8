"""Sampling and one-row-at-a-time oracle helpers of the full-size parity tests."""

import numpy as np

from g4inputs import gen
from oracle import norm_rope as onr

f64 = gen.to_f64

# The prologue hands q and k to attention as bf16 (half-ulp 2^-9 relative),
# while the oracle keeps them in fp64, so each logit scale * q.k moves by up
# to about 2^-8 |scale q.k|: 0.01 for the largest logits here (about 2.5 in
# magnitude for RMS-normalised rows with N(1, 0.1) weights and random
# directions, up to ~4 in the tails).  The log-sum-exp is a weighted mean of
# the logits' errors, so it gets the same bound.
LSE_ATOL = 1e-2


def sample_tokens(S, window, n_rand, seed):
    """First/last tokens, 32-key tile edges, window edges and seeded random positions."""
    fixed = {0, 1, 31, 32, 33, 127, 128, S // 2, S - 2, S - 1}
    if window:
        fixed |= {window - 1, window, window + 1, min(S - 1, 2 * window + 5)}
    rng = np.random.default_rng(seed)
    rand = set(rng.integers(0, S, size=n_rand).tolist())
    return np.array(sorted(t for t in fixed | rand if 0 <= t < S), dtype=np.int64)


def prefill_oracle_rows(s, b, g, toks, heads):
    """Oracle out [len(toks), len(heads), D] and lse for batch b, KV group g."""
    c = s["c"]
    slo, shi = gen.image_spans(c.S, c.images)
    hi = int(max(toks.max(), shi[toks].max())) + 1
    lo = 0 if c.window == 0 else max(0, int(min(toks.min() - c.window + 1, slo[toks].min())))
    pos_k = np.arange(lo, hi)[None, :]
    if c.k_eq_v:
        X = f64(s["X"][b:b + 1, lo:hi, g:g + 1])
        K, V = onr.kv_tied_k_v(X, f64(s["wk"]), pos_k, c.rotary_dims, c.theta)
    else:
        K = onr.norm_rope(f64(s["k_raw"][b:b + 1, lo:hi, g:g + 1]), f64(s["wk"]), pos_k, c.rotary_dims, c.theta)
        V = onr.norm_rope(f64(s["v_raw"][b:b + 1, lo:hi, g:g + 1]), None, pos_k, 0, c.theta)
    out = np.zeros((len(toks), len(heads), c.D))
    lse = np.zeros((len(toks), len(heads)))
    for ti, t in enumerate(toks):
        qraw = f64(s["q_raw"][b:b + 1, t:t + 1, heads])                 # [1, 1, H, D]
        q = onr.norm_rope(qraw, f64(s["wq"]), np.array([[t]]), c.rotary_dims, c.theta)
        k0 = 0 if c.window == 0 else max(0, int(t) - c.window + 1)
        # visible keys of row t: its window (or every earlier key), plus its image block
        keys = sorted(set(range(k0, int(t) + 1)) | set(range(int(slo[t]), int(shi[t]) + 1)))
        kk = K[0, np.asarray(keys) - lo, 0]
        vv = V[0, np.asarray(keys) - lo, 0]
        for hi_, _ in enumerate(heads):
            sc = c.scale * (kk @ q[0, 0, hi_])
            m = sc.max()
            e = np.exp(sc - m)
            out[ti, hi_] = (e @ vv) / e.sum()
            lse[ti, hi_] = m + np.log(e.sum())
    return out, lse
