"""Host-side logic of bench.py checked against the oracle's masks (no GPU)."""

import numpy as np
import pytest

import bench
from g4inputs import gen
from oracle import attention as oat


@pytest.mark.parametrize("S,w,images", [(50, 8, [(3, 5), (20, 25)]), (64, 0, [(0, 10), (30, 34)]),
                                        (100, 16, []), (300, 64, [(0, 20), (40, 150), (250, 50)])])
def test_span_pair_count_matches_the_mask(S, w, images):
    lo, hi = gen.image_spans(S, images)
    assert bench.span_pairs(S, w, lo, hi) == int(oat.mask_spans(S, w, lo, hi).sum())


def test_image_spans_layout():
    lo, hi = gen.image_spans(12, [(2, 3), (9, 3)])
    assert lo.tolist() == [0, 1, 2, 2, 2, 5, 6, 7, 8, 9, 9, 9]
    assert hi.tolist() == [0, 1, 4, 4, 4, 5, 6, 7, 8, 11, 11, 11]


@pytest.mark.parametrize("S,w", [(1024, 512), (8192, 0), (16384, 1024), (5, 8), (100, 1), (3000, 700)])
def test_visible_pair_count_matches_the_mask(S, w):
    assert bench.visible_pairs(S, w) == oat.visible_pairs(S, w)


def test_cpu_baseline_runs_on_small_stand_ins(monkeypatch):
    """The per-config oracle baseline runs end to end (on tiny CPU stand-ins for the workloads) and
    reports every config with its sample, the host's cores and a positive rate."""
    import dataclasses
    import torch
    from g4inputs import WORKLOADS

    monkeypatch.setattr(torch.cuda, "synchronize", lambda *a, **k: None)
    W = {k: dataclasses.replace(v, S=min(v.S, 96), B=1) for k, v in WORKLOADS.items()}

    def prefill(c):
        s = dict(c=c, q_raw=gen.normal_bf16((c.B, c.S, c.Hq, c.D), (9, c.cfg_id, 1, 0)),
                 wq=gen.norm_weight(c.D, (9, c.cfg_id, 2, 0)), wk=gen.norm_weight(c.D, (9, c.cfg_id, 3, 0)))
        if c.k_eq_v:
            s["X"] = gen.normal_bf16((c.B, c.S, c.Hkv, c.D), (9, c.cfg_id, 4, 0))
        else:
            s["k_raw"] = gen.normal_bf16((c.B, c.S, c.Hkv, c.D), (9, c.cfg_id, 5, 0))
            s["v_raw"] = gen.normal_bf16((c.B, c.S, c.Hkv, c.D), (9, c.cfg_id, 6, 0))
        return s

    cd = dataclasses.replace(WORKLOADS["31b_global_kv_decode"], B=2)
    n = np.array([70, 33])
    st = {"e2b_sliding": prefill(W["e2b_sliding_prefill"]), "e2b_global": prefill(W["e2b_global_prefill"]),
          "sliding": prefill(W["31b_sliding_prefill"]), "global": prefill(W["31b_global_kv_prefill"]),
          "decode": dict(c=cd, n=n, L=n - 1, cache=gen.normal_bf16((2, cd.Hkv, 70, cd.D), (9, 5, 7, 0)),
                         q_raw=gen.normal_bf16((2, 1, cd.Hq, cd.D), (9, 5, 8, 0)),
                         wq=gen.norm_weight(cd.D, (9, 5, 9, 0)))}
    out = bench.cpu_baseline(torch, gen, st, lambda m: None, budget_s=0.5)
    assert out["kind"] == "oracle" and out["unit"] == "TFLOP/s" and out["value"] > 0
    assert out["cores"] >= 1
    assert set(out["per_config"]) == {"e2b_sliding_prefill", "e2b_global_prefill", "31b_sliding_prefill",
                                      "31b_global_kv_prefill", "31b_global_kv_decode"}
    assert all(v["value"] > 0 and v["sample"] for v in out["per_config"].values())


def test_bench_refuses_more_than_one_gpu():
    """One GPU only: --gpus N > 1 exits non-zero with a message, before touching a GPU."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], cwd=root,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "one GPU" in r.stderr
