"""Pin the model shapes with the KV-cache sizes the PyTorch port prints."""

import json
import os

import pytest

from oracle import kv_cache as kc

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "kv_cache_sizes.json")))


@pytest.mark.parametrize("model", sorted(GOLD["models"]))
def test_printed_cache_sizes(model):
    m = GOLD["models"][model]
    args = dict(num_layers=m["num_layers"], local_per_global=m["local_per_global"],
                kv_heads=m["kv_heads"], global_kv_heads=m["global_kv_heads"],
                head_dim=m["head_dim"], global_head_dim=m["global_head_dim"],
                context=GOLD["context"])
    full = kc.kv_cache_bytes(**args) / 1e9
    win = kc.kv_cache_bytes(window=m["window"], **args) / 1e9
    assert round(full, 1) == m["printed_full_GB"]
    assert round(win, 1) == m["printed_windowed_GB"]


def test_planted_single_tensor_kv_fails():
    # Storing one tensor on the K=V global layers would not give the printed 29.5 GB.
    n_local, n_global = kc.layer_split(60, 5)
    assert (n_local, n_global) == (50, 10)
    one_tensor = (2 * 2 * 50 * 16 * 256 * 32768 + 1 * 2 * 10 * 4 * 512 * 32768) / 1e9
    assert round(one_tensor, 1) != 29.5
    # nor would 256-wide global heads
    narrow = kc.kv_cache_bytes(60, 5, 16, 4, 256, 256, 32768) / 1e9
    assert round(narrow, 1) != 29.5
