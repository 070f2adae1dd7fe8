"""Decode of a K=V global layer over its raw-projection cache (g4attn_kv_tied_append +
g4attn_decode_tied) against the fp64 oracle through the C ABI."""

import numpy as np
import pytest
import torch

from g4inputs import gen
from oracle import attention as oat
from oracle import norm_rope as onr
from tests._cmp import assert_parity

pytestmark = pytest.mark.gpu

DEV = "cuda"
f64 = gen.to_f64
D, ROT, THETA = 512, 128, 1e6


def _bf(shape, seed):
    return gen.normal_bf16(shape, (7, 111, seed, 0), "cpu").to(DEV)


def _caches(B, Hkv, cap):
    xc = torch.full((B, Hkv, cap, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    rc = torch.full((B, Hkv, cap), float("nan"), dtype=torch.float32, device=DEV)
    kc = torch.full((B, Hkv, cap, ROT), float("nan"), dtype=torch.bfloat16, device=DEV)
    return xc, rc, kc


def test_kv_tied_append_rows(gpu_lib):
    """X is copied bit for bit; r and the rotated key part match the oracle at each row's position."""
    g4 = gpu_lib
    B, S, Hkv, cap = 2, 40, 4, 100
    X = _bf((B, S, Hkv, D), 1)
    wk = gen.norm_weight(D, (7, 111, 2, 0)).to(DEV)
    xc, rc, kc = _caches(B, Hkv, cap)
    pos0 = torch.tensor([0, 55], dtype=torch.int32, device=DEV)
    g4.g4attn_kv_tied_append(X, wk, xc, rc, kc, THETA, pos0=pos0, max_pos=55 + S - 1)
    torch.cuda.synchronize()
    for b, p0 in enumerate((0, 55)):
        assert torch.equal(xc[b, :, p0:p0 + S], X[b].permute(1, 0, 2))
        pos = np.arange(p0, p0 + S)[None, :]
        xb = f64(X[b:b + 1])
        np.testing.assert_allclose(rc[b, :, p0:p0 + S].cpu().numpy(), onr.inv_rms(xb)[0].transpose(1, 0), rtol=2e-6)
        krot = onr.apply_rope(xb * f64(wk), pos, ROT, THETA)                 # before r
        want = np.concatenate([krot[..., :64], krot[..., 256:320]], axis=-1)[0].transpose(1, 0, 2)
        assert_parity(f64(kc[b, :, p0:p0 + S]), want, "Krot rows")
    assert bool(torch.isnan(xc[0, :, S:]).all()) and bool(torch.isnan(rc[1, :, :55]).all())


@pytest.mark.parametrize("Hq,Hkv,splits", [(32, 4, 0), (8, 1, 3), (16, 2, 1), (16, 1, 0), (16, 1, 2)])
def test_decode_tied_vs_oracle(gpu_lib, Hq, Hkv, splits):
    g4 = gpu_lib
    lens = [1, 17, 300, 1029, 64]
    B, cap = len(lens), 1100
    X = _bf((B, max(lens), Hkv, D), 10 + splits)
    wk = gen.norm_weight(D, (7, 111, 11, 0)).to(DEV)
    wq = gen.norm_weight(D, (7, 111, 12, 0)).to(DEV)
    xc, rc, kc = _caches(B, Hkv, cap)
    g4.g4attn_kv_tied_append(X, wk, xc, rc, kc, THETA)       # positions 0.. of every sequence
    qraw = _bf((B, 1, Hq, D), 13)
    q = torch.empty_like(qraw)
    last = torch.tensor([n - 1 for n in lens], dtype=torch.int32, device=DEV)
    g4.g4attn_norm_rope(qraw, q, wq, D, ROT, THETA, pos0=last)
    desc = g4.layer_desc(Hq, Hkv, D, k_eq_v=True, rotary_dims=ROT, rope_theta=THETA)
    out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=DEV)
    kv_len = torch.tensor(lens, dtype=torch.int32, device=DEV)
    g4.g4attn_decode_tied(desc, q.view(B, Hq, D), xc, rc, kc, wk, kv_len, max(lens), out, lse=lse,
                          num_splits=splits)
    torch.cuda.synchronize()
    K, V = onr.kv_tied_k_v(f64(X), f64(wk), np.tile(np.arange(max(lens)), (B, 1)), ROT, THETA)
    kcache = K.transpose(0, 2, 1, 3)      # [B, Hkv, S, D]
    vcache = V.transpose(0, 2, 1, 3)
    qo = onr.norm_rope(f64(qraw), f64(wq), np.array(lens)[:, None] - 1, ROT, THETA)[:, 0]
    ro, rl = oat.decode_attention(qo, kcache, vcache, np.array(lens), desc.scale)
    assert_parity(f64(out), ro, f"K=V decode Hq={Hq} Hkv={Hkv} splits={splits}")
    # the oracle's q and keys are fp64 from the raw inputs; the GPU's q passes the prologue in bf16 and
    # carries w_k on its unrotated dims in bf16: up to ~2^-8 of each logit (~2 here), as in the
    # full-size tests
    np.testing.assert_allclose(lse.cpu().numpy(), rl, rtol=0, atol=1e-2)


def test_decode_tied_equals_prefill_last_row(gpu_lib):
    """Decoding the last token over the raw-projection cache matches the K=V prefill's last row."""
    g4 = gpu_lib
    B, S, Hq, Hkv = 1, 777, 32, 4
    X = _bf((B, S, Hkv, D), 20)
    q = _bf((B, S, Hq, D), 21)
    wk = gen.norm_weight(D, (7, 111, 22, 0)).to(DEV)
    desc = g4.layer_desc(Hq, Hkv, D, k_eq_v=True, rotary_dims=ROT, rope_theta=THETA)
    pre = torch.empty_like(q)
    g4.g4attn_prefill(desc, q, X, None, pre, w_k=wk)
    xc, rc, kc = _caches(B, Hkv, S)
    g4.g4attn_kv_tied_append(X, wk, xc, rc, kc, THETA)
    out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=DEV)
    g4.g4attn_decode_tied(desc, q[:, S - 1].contiguous(), xc, rc, kc, wk,
                          torch.tensor([S], dtype=torch.int32, device=DEV), S, out)
    torch.cuda.synchronize()
    assert_parity(f64(out[0]), f64(pre[0, S - 1]), "K=V decode vs prefill last row")


def test_kv_shared_layers_reuse_one_cache(gpu_lib):
    """KV-shared layers: a later layer decodes over an earlier layer's caches by passing the same
    tensors; the result is bit-identical to decoding over private copies, and the shared caches
    are left untouched."""
    g4 = gpu_lib
    B, Hq, Hkv, Dh, cap = 3, 8, 2, 256, 600
    lens = torch.tensor([5, 333, 600], dtype=torch.int32, device=DEV)
    kc, vc = _bf((B, Hkv, cap, Dh), 30), _bf((B, Hkv, cap, Dh), 31)
    before = (kc.clone(), vc.clone())
    desc = g4.layer_desc(Hq, Hkv, Dh, rotary_dims=Dh)
    outs = []
    for layer in range(2):                               # two layers, one pair of caches
        q = _bf((B, Hq, Dh), 40 + layer)
        shared = torch.empty((B, Hq, Dh), dtype=torch.bfloat16, device=DEV)
        private = torch.empty_like(shared)
        g4.g4attn_decode(desc, q, kc, vc, lens, cap, shared)
        g4.g4attn_decode(desc, q, kc.clone(), vc.clone(), lens, cap, private)
        torch.cuda.synchronize()
        assert torch.equal(shared, private)
        outs.append(shared)
    assert torch.equal(kc, before[0]) and torch.equal(vc, before[1])
    assert not torch.equal(outs[0], outs[1])
