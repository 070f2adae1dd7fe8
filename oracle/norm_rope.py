"""fp64 oracle for the attention prologue: plain-weight RMSNorm + RoPE.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources
-------
* Plain-weight RMSNorm: the norm weight multiplies the normalised vector
  directly, without the ``1 + w`` offset of earlier Gemma generations
  [Gemma 4 Keras docs, "What changed from Gemma 3"; gemma4-pt-claude README,
  "Attention Backend Notes" (multiplicative norms, one-initialised)].
* QK-norm and V-norm: every variant normalises queries, keys and values
  [gemma4-pt-claude README, "Supported Models" and "Key architectural
  features"].  The V-norm carries no weight (reading: the value norm is
  weightless; the 31B K=V workload states it).
* RoPE: each 2-D subspace is rotated by the 2x2 rotation matrix of angle
  ``position * frequency`` [vinija.ai Gemma 4 primer, "Dual RoPE
  configurations", rotation-matrix equation].  Sliding layers rotate every
  pair; global layers rotate only ``partial_rotary_factor`` (0.25) of each
  head and pass the rest through ("zero-pad partial rope")
  [Gemma 4 Keras docs, "What changed from Gemma 3" and the ``Gemma4Model``
  argument table, ``partial_rotary_factor``].

Readings where the pages are silent
-----------------------------------
* Pairing is rotate-half: dimension ``j`` pairs with ``j + D/2``.
* Frequencies: ``inv_freq_j = theta ** (-2 j / D)`` for ``j < rotary_dims/2``
  and ``0`` for the remaining pairs (zero padding), with denominator the full
  head width ``D``; theta 1e4 on sliding layers, 1e6 on global layers.
* Order: normalise, multiply by the weight, then rotate.
* RMSNorm epsilon 1e-6, added to the mean square inside the square root.

Pins (tests/test_oracle_norm_rope.py)
-------------------------------------
* RMSNorm vs ``torch.nn.functional.rms_norm`` in float64 (a library routine);
  closed forms: weightless output has mean square ``ms / (ms + eps)``,
  ``w = 0`` gives exact zeros, scale invariance.
* RoPE vs complex multiplication ``(x_j + i x_{j+D/2}) * exp(i p f_j)`` (the
  primer writes RoPE as ``x * e^{i theta}``); invariants: pair norms kept,
  pass-through dims bit-identical, position 0 is the identity, and the
  relative-position identity ``<R_m q, R_n k> = <R_{m-n} q, k>``.
"""

import numpy as np

RMS_EPS = 1e-6


def rms_norm(x, weight=None, eps=RMS_EPS):
    """``y = x / sqrt(mean_D(x^2) + eps) * w`` over the last axis, in fp64.

    ``weight=None`` is the weightless V-norm.  The weight is applied as is
    (plain weight, no ``1 + w``).
    """
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    y = x / np.sqrt(ms + eps)
    if weight is not None:
        y = y * np.asarray(weight, dtype=np.float64)
    return y


def inv_rms(x, eps=RMS_EPS):
    """The per-row factor ``1 / sqrt(mean_D(x^2) + eps)`` (fp64)."""
    x = np.asarray(x, dtype=np.float64)
    return 1.0 / np.sqrt(np.mean(x * x, axis=-1) + eps)


def rope_inv_freq(head_dim, rotary_dims, theta):
    """Per-pair angular frequencies, zero-padded past ``rotary_dims / 2``.

    Pair ``j`` (dims ``j`` and ``j + head_dim/2``) turns at
    ``theta ** (-2 j / head_dim)`` when ``j < rotary_dims / 2`` and not at all
    otherwise, so the live frequencies of a partial rotation are exactly those
    of a full rotation of the same head width.
    """
    half = head_dim // 2
    j = np.arange(half, dtype=np.float64)
    f = np.power(float(theta), -2.0 * j / float(head_dim))
    f[rotary_dims // 2:] = 0.0
    return f


def apply_rope(x, positions, rotary_dims, theta):
    """Rotate pairs ``(j, j + D/2)`` of ``x[..., S, H, D]`` by ``p * f_j``.

    ``positions`` has shape ``[..., S]`` (integers).  A pair with zero
    frequency is copied unchanged, which is the pass-through part of a
    partial rotation.
    """
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    half = D // 2
    f = rope_inv_freq(D, rotary_dims, theta)
    pos = np.asarray(positions, dtype=np.float64)
    ang = pos[..., None] * f                      # [..., S, half]
    c = np.cos(ang)[..., None, :]                 # broadcast over heads
    s = np.sin(ang)[..., None, :]
    a = x[..., :half]
    b = x[..., half:]
    y = np.empty_like(x)
    y[..., :half] = a * c - b * s
    y[..., half:] = b * c + a * s
    # Pairs that do not turn are passed through exactly (cos 0 = 1, sin 0 = 0
    # already give this; the copy makes the pass-through explicit).
    live = rotary_dims // 2
    y[..., live:half] = a[..., live:]
    y[..., half + live:] = b[..., live:]
    return y


def norm_rope(x, weight, positions, rotary_dims, theta, eps=RMS_EPS):
    """Prologue of one projection: RMSNorm (optional weight) then RoPE.

    ``x``: ``[B, S, H, D]``; ``positions``: ``[B, S]``.  ``rotary_dims = 0``
    skips the rotation (the V-norm).
    """
    y = rms_norm(x, weight, eps)
    if rotary_dims:
        y = apply_rope(y, positions, rotary_dims, theta)
    return y


def kv_tied_k_v(x, w_k, positions, rotary_dims, theta, eps=RMS_EPS):
    """K and V of a global K=V layer from the one tied projection ``x``.

    Key and value projections share weights on global layers of the dense
    and MoE sizes [Gemma 4 Keras docs, "What changed from Gemma 3", K=V
    global MQA; gemma4-pt-claude README, "Key architectural features", K=V].
    The key takes the weighted K-norm and RoPE; the value takes the
    weightless V-norm and no rotation.
    """
    k = norm_rope(x, w_k, positions, rotary_dims, theta, eps)
    v = norm_rope(x, None, positions, 0, theta, eps)
    return k, v
