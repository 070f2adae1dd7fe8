"""Seeded, chunk-deterministic random inputs.

Every tensor is keyed by ``(seed, cfg_id, tensor_id, chunk)``:

* on the host, ``numpy.random.default_rng(SeedSequence(key))`` draws fp32
  standard normals which torch rounds to bfloat16 (round-to-nearest-even);
* on a GPU, a ``torch.Generator`` on that device seeded from the same key
  draws the fp32 normals (used for tensors too large to draw on the host,
  e.g. a 17 GB decode cache).  Host and device draws of one key differ; a
  test always hands the oracle the exact bf16 values the kernels saw.

Norm weights are ``1 + 0.1 * N(0, 1)`` rounded to bf16.
"""

import numpy as np
import torch

# tensor ids
Q, K, V, X, WQ, WK, CACHE, QDEC, LENS, CACHE_V = range(10)  # CACHE_V: separate V cache


def seed_key(cfg_id, tensor_id, chunk=0, seed=0):
    return (int(seed), int(cfg_id), int(tensor_id), int(chunk))


def _seed_int(key):
    return int(np.random.SeedSequence(list(key)).generate_state(1, np.uint64)[0] >> 1)


def normal_bf16(shape, key, device="cpu", scale=1.0):
    """bf16 tensor of ``scale * N(0, 1)`` draws keyed by ``key``."""
    if str(device) == "cpu":
        rng = np.random.default_rng(np.random.SeedSequence(list(key)))
        a = rng.standard_normal(size=shape, dtype=np.float32)
        if scale != 1.0:
            a *= np.float32(scale)
        return torch.from_numpy(a).to(torch.bfloat16)
    g = torch.Generator(device=device)
    g.manual_seed(_seed_int(key))
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if scale != 1.0:
        t.mul_(scale)
    return t.to(torch.bfloat16)


def norm_weight(D, key):
    """Norm weight ``1 + 0.1 N(0,1)`` as bf16 (host)."""
    rng = np.random.default_rng(np.random.SeedSequence(list(key)))
    a = 1.0 + 0.1 * rng.standard_normal(size=(D,), dtype=np.float32)
    return torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16)


def decode_lengths(B, lo, hi, key):
    """Cache lengths drawn uniformly from ``[lo, hi]`` (both ends included)."""
    rng = np.random.default_rng(np.random.SeedSequence(list(key)))
    return rng.integers(lo, hi, size=B, endpoint=True).astype(np.int32)


def to_f64(t):
    """Exact widening of a (bf16) torch tensor to a float64 numpy array."""
    return t.detach().to("cpu").to(torch.float32).numpy().astype(np.float64)


def image_spans(S, images):
    """Per-row bidirectional span bounds of one sequence with image blocks at
    ``(start, length)``: rows of a block get the block's first and last
    position, text rows their own position.  int32 arrays [S]."""
    lo = np.arange(S, dtype=np.int32)
    hi = np.arange(S, dtype=np.int32)
    for st, n in images:
        lo[st:st + n] = st
        hi[st:st + n] = st + n - 1
    return lo, hi
