"""Comparison helpers for the GPU-vs-oracle parity tests (test code only)."""

import numpy as np

# Parity bar for bf16 outputs against the fp64 oracle.
MAX_ABS = 2e-2
REL_L2 = 5e-3


def errors(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    d = got - ref
    max_abs = float(np.max(np.abs(d))) if d.size else 0.0
    den = float(np.sqrt(np.sum(ref * ref)))
    rel = float(np.sqrt(np.sum(d * d)) / den) if den > 0 else float(np.sqrt(np.sum(d * d)))
    return max_abs, rel


def assert_parity(got, ref, what="", max_abs=MAX_ABS, rel_l2=REL_L2):
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    ma, rel = errors(got, ref)
    assert ma <= max_abs and rel <= rel_l2, f"{what}: max-abs {ma:.3e} rel-L2 {rel:.3e}"
    return ma, rel
