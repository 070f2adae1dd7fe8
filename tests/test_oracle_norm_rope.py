"""Pins for the fp64 prologue oracle (RMSNorm + RoPE); CPU only."""

import numpy as np
import pytest
import torch

from oracle import norm_rope as nr

RNG = np.random.default_rng(1234)


def _x(*shape):
    return RNG.standard_normal(shape)


# ---------------------------------------------------------------- RMSNorm
@pytest.mark.parametrize("D", [8, 256, 512])
@pytest.mark.parametrize("weighted", [True, False])
def test_rmsnorm_matches_torch_library(D, weighted):
    x = _x(3, 5, 2, D)
    w = 1.0 + 0.1 * _x(D) if weighted else None
    ref = torch.nn.functional.rms_norm(
        torch.from_numpy(x), (D,), None if w is None else torch.from_numpy(w), eps=nr.RMS_EPS)
    np.testing.assert_allclose(nr.rms_norm(x, w), ref.numpy(), rtol=1e-13, atol=1e-13)


def test_rmsnorm_closed_forms():
    x = _x(64, 512) * 3.0
    ms = np.mean(x * x, axis=-1)
    y = nr.rms_norm(x, None)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), ms / (ms + nr.RMS_EPS), rtol=1e-13)
    # plain weight: w = 0 gives exact zeros (a 1 + w offset would not)
    assert np.all(nr.rms_norm(x, np.zeros(512)) == 0.0)
    # w = 1 is the weightless norm
    np.testing.assert_array_equal(nr.rms_norm(x, np.ones(512)), y)
    # scale invariance when eps = 0
    np.testing.assert_allclose(nr.rms_norm(7.5 * x, None, eps=0.0), nr.rms_norm(x, None, eps=0.0),
                               rtol=1e-13)


@pytest.mark.parametrize("D,scale", [(512, 1.0), (512, 40.0), (256, 0.01)])
def test_inv_rms_matches_torch_library(D, scale):
    """inv_rms is the factor torch's rms_norm applies: rms_norm(x) / x, element by
    element (a library routine, not the oracle's own formula)."""
    x = _x(4, 33, D) * scale
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (D,), None, eps=nr.RMS_EPS).numpy()
    r = nr.inv_rms(x)
    assert r.shape == x.shape[:-1]
    np.testing.assert_allclose(r[..., None] * x, ref, rtol=1e-13, atol=1e-13 * scale)
    np.testing.assert_allclose(ref[..., 5] / x[..., 5], r, rtol=1e-12)
    # and the factor rescales the weightless norm of the oracle itself
    np.testing.assert_allclose(r[..., None] * x, nr.rms_norm(x, None), rtol=1e-14)


# ---------------------------------------------------------------- RoPE
def _rope_complex(x, pos, rotary_dims, theta):
    """RoPE written as complex multiplication x * e^{i p f} on pairs (j, j + D/2)."""
    D = x.shape[-1]
    h = D // 2
    z = x[..., :h] + 1j * x[..., h:]
    f = np.array([theta ** (-(2.0 * j) / D) if j < rotary_dims // 2 else 0.0 for j in range(h)])
    ph = np.exp(1j * pos[..., None, None] * f)   # [..., S, 1, h]
    zr = z * ph
    return np.concatenate([zr.real, zr.imag], axis=-1)


@pytest.mark.parametrize("D,rot,theta", [(256, 256, 1e4), (512, 128, 1e6), (512, 512, 1e6), (16, 4, 1e4)])
def test_rope_matches_complex_multiplication(D, rot, theta):
    x = _x(2, 7, 3, D)
    pos = np.array([[0, 1, 2, 5, 511, 4097, 131072], [3, 9, 1000, 32767, 32768, 65535, 100000]])
    # Angles reach 1.3e5 rad: one ulp of frequency there moves the angle by
    # ~3e-11, so agreement is to 1e-9, not to the last bit.
    np.testing.assert_allclose(nr.apply_rope(x, pos, rot, theta), _rope_complex(x, pos, rot, theta),
                               rtol=0, atol=1e-9)


def test_rope_frequencies():
    # The live frequencies of a partial rotation equal those of the full one.
    full = nr.rope_inv_freq(512, 512, 1e6)
    part = nr.rope_inv_freq(512, 128, 1e6)
    assert np.count_nonzero(part) == 64 and np.all(part[64:] == 0.0)
    np.testing.assert_array_equal(part[:64], full[:64])
    assert full[0] == 1.0
    # geometric progression with ratio theta^(-2/D)
    np.testing.assert_allclose(full[1:] / full[:-1], 1e6 ** (-2.0 / 512), rtol=1e-12)
    # pair 0 turns by exactly p radians
    x = np.zeros((1, 1, 1, 512)); x[..., 0] = 1.0
    y = nr.apply_rope(x, np.array([[3]]), 128, 1e6)
    assert abs(y[0, 0, 0, 0] - np.cos(3.0)) < 1e-15 and abs(y[0, 0, 0, 256] - np.sin(3.0)) < 1e-15


@pytest.mark.parametrize("D,rot", [(256, 256), (512, 128)])
def test_rope_invariants(D, rot):
    x = _x(1, 6, 4, D)
    pos = np.array([[0, 1, 17, 1023, 32768, 131072]])
    y = nr.apply_rope(x, pos, rot, 1e6)
    h = D // 2
    # pair norms are preserved
    np.testing.assert_allclose(y[..., :h] ** 2 + y[..., h:] ** 2, x[..., :h] ** 2 + x[..., h:] ** 2,
                               rtol=1e-12)
    # pass-through dims are bit-identical
    live = rot // 2
    np.testing.assert_array_equal(y[..., live:h], x[..., live:h])
    np.testing.assert_array_equal(y[..., h + live:], x[..., h + live:])
    # position 0 is the identity
    np.testing.assert_array_equal(y[:, 0], x[:, 0])


@pytest.mark.parametrize("D,rot,theta", [(256, 256, 1e4), (512, 128, 1e6)])
def test_rope_relative_position(D, rot, theta):
    q = _x(1, 1, 1, D)
    k = _x(1, 1, 1, D)
    for m, n in [(5, 2), (1000, 999), (70000, 3), (12, 40)]:
        lhs = np.sum(nr.apply_rope(q, np.array([[m]]), rot, theta) * nr.apply_rope(k, np.array([[n]]), rot, theta))
        rhs = np.sum(nr.apply_rope(q, np.array([[m - n]]), rot, theta) * k)
        assert abs(lhs - rhs) < 1e-9 * max(1.0, abs(rhs))


def test_norm_rope_order_and_kv_tying():
    x = _x(2, 5, 2, 512)
    w = 1.0 + 0.1 * _x(512)
    pos = np.tile(np.arange(5), (2, 1))
    y = nr.norm_rope(x, w, pos, 128, 1e6)
    np.testing.assert_array_equal(y, nr.apply_rope(nr.rms_norm(x, w), pos, 128, 1e6))
    # K=V tying: with unit K weight and no rotation, K and V are the same tensor
    k, v = nr.kv_tied_k_v(x, np.ones(512), pos, 0, 1e6)
    np.testing.assert_array_equal(k, v)
    k, v = nr.kv_tied_k_v(x, w, pos, 128, 1e6)
    np.testing.assert_array_equal(v, nr.rms_norm(x, None))


# ----------------------------------------------- planted mistakes are caught
def test_planted_rope_mistakes_fail_the_pins():
    x = _x(1, 3, 1, 256)
    pos = np.array([[1, 7, 300]])
    ref = _rope_complex(x, pos, 256, 1e4)

    def wrong_sign(x, pos, rot, theta):
        y = nr.apply_rope(x, -pos, rot, theta)   # clockwise rotation
        return y

    def interleaved_pairs(x, pos, rot, theta):  # pairs (2j, 2j+1) instead of (j, j+D/2)
        D = x.shape[-1]
        perm = np.concatenate([np.arange(0, D, 2), np.arange(1, D, 2)])
        inv = np.argsort(perm)
        return nr.apply_rope(x[..., perm], pos, rot, theta)[..., inv]

    for bad in (wrong_sign, interleaved_pairs):
        assert not np.allclose(bad(x, pos, 256, 1e4), ref, atol=1e-6)


def test_planted_norm_offset_fails_the_pin():
    x = _x(4, 512)
    gemma3_style = nr.rms_norm(x, None) * (1.0 + np.zeros(512))   # 1 + w with w = 0
    assert not np.all(gemma3_style == 0.0)   # the w = 0 -> 0 pin would fail for it
