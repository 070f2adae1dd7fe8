"""Bidirectional image spans (span_lo / span_hi of g4attn_prefill and g4attn_prefill_chunk) against
the fp64 oracle through the C ABI: blocks at the start and end of a sequence, longer than the
window, crossing tiles, single-token blocks, with chunked rows over caches."""

import numpy as np
import pytest
import torch

from g4inputs import gen
from oracle import attention as oat
from tests._cmp import assert_parity

pytestmark = pytest.mark.gpu

DEV = "cuda"
f64 = gen.to_f64
LAYOUTS = [[(0, 20), (40, 150), (250, 50)], [(31, 2), (63, 66), (140, 1)]]


def _bf(shape, seed):
    return gen.normal_bf16(shape, (7, 99, seed, 0), "cpu").to(DEV)


def _span_tensors(S, layouts):
    lo = np.stack([gen.image_spans(S, im)[0] for im in layouts])
    hi = np.stack([gen.image_spans(S, im)[1] for im in layouts])
    return lo, hi, torch.from_numpy(lo).to(DEV), torch.from_numpy(hi).to(DEV)


@pytest.mark.parametrize("D,w,Hq,Hkv", [(256, 64, 8, 2), (512, 0, 8, 1), (256, 0, 4, 1), (512, 100, 8, 2)])
def test_prefill_spans_vs_oracle(gpu_lib, D, w, Hq, Hkv):
    g4 = gpu_lib
    B, S = 2, 300
    q, k, v = _bf((B, S, Hq, D), 1), _bf((B, S, Hkv, D), 2), _bf((B, S, Hkv, D), 3)
    lo, hi, tlo, thi = _span_tensors(S, LAYOUTS)
    desc = g4.layer_desc(Hq, Hkv, D, window=w, rotary_dims=D)
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=DEV)
    g4.g4attn_prefill(desc, q, k, v, out, lse=lse, span_lo=tlo, span_hi=thi)
    torch.cuda.synchronize()
    for b in range(B):
        m = oat.mask_spans(S, w, lo[b], hi[b])
        ro, rl = oat.attention_masked(f64(q[b:b + 1]), f64(k[b:b + 1]), f64(v[b:b + 1]), desc.scale, m)
        assert_parity(f64(out[b:b + 1]), ro, f"spans D={D} w={w} b={b}")
        np.testing.assert_allclose(lse[b:b + 1].cpu().numpy(), rl, rtol=0, atol=2e-3)


def test_prefill_chunk_spans_equal_whole_sequence(gpu_lib):
    """Spans given in absolute positions survive the chunked path over caches."""
    g4 = gpu_lib
    B, S, Hq, Hkv, D, w, chunk = 2, 300, 8, 2, 256, 64, 100
    q, k, v = _bf((B, S, Hq, D), 4), _bf((B, S, Hkv, D), 5), _bf((B, S, Hkv, D), 6)
    lo, hi, tlo, thi = _span_tensors(S, LAYOUTS)
    desc = g4.layer_desc(Hq, Hkv, D, window=w, rotary_dims=D)
    kc = k.permute(0, 2, 1, 3).contiguous()
    vc = v.permute(0, 2, 1, 3).contiguous()
    out = torch.empty_like(q)
    ql = torch.full((B,), chunk, dtype=torch.int32, device=DEV)
    for c0 in range(0, S, chunk):
        p0 = torch.full((B,), c0, dtype=torch.int32, device=DEV)
        oo = torch.empty((B, chunk, Hq, D), dtype=torch.bfloat16, device=DEV)
        # the chunk's rows carry their (absolute) span bounds; keys past the chunk are not cached yet
        g4.g4attn_prefill_chunk(desc, q[:, c0:c0 + chunk].contiguous(), kc, vc, oo, p0, ql, c0 + chunk - 1,
                                span_lo=tlo[:, c0:c0 + chunk].contiguous(), span_hi=thi[:, c0:c0 + chunk].contiguous())
        out[:, c0:c0 + chunk] = oo
    torch.cuda.synchronize()
    for b in range(B):
        # a chunk's rows see their block only up to the chunk's last position (the keys cached so far)
        hic = np.minimum(hi[b], (np.arange(S) // chunk) * chunk + chunk - 1)
        m = oat.mask_spans(S, w, lo[b], hic)
        ro, _ = oat.attention_masked(f64(q[b:b + 1]), f64(k[b:b + 1]), f64(v[b:b + 1]), desc.scale, m)
        assert_parity(f64(out[b:b + 1]), ro, f"chunked spans b={b}")
