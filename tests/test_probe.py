"""The roofline probes (libg4probe.so): exports and host-side argument checks
on the CPU; on the GPU, that the streaming read touches every byte once and
that the MFMA loop runs the requested number of rounds."""

import ctypes
import os
import re

import numpy as np
import pytest

from decoder_attention_g4attn_amd import probe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "g4probe.h")

built = pytest.mark.skipif(not os.path.exists(probe.PROBE_LIB_PATH), reason="libg4probe.so not built")
FAKE = ctypes.c_void_p(0x100000)


@built
def test_exports_every_declared_probe():
    lib = probe.load()
    decl = set(re.findall(r"^int\s+(g4probe_\w+)\s*\(", open(HEADER).read(), flags=re.M))
    assert decl == {"g4probe_mfma_bf16", "g4probe_stream_read"}
    for name in decl:
        assert hasattr(lib, name)


@built
def test_invalid_arguments_launch_nothing():
    lib = probe.load()
    assert lib.g4probe_mfma_bf16(None, 1, 1, 0, None) == -1
    assert lib.g4probe_mfma_bf16(FAKE, 0, 1, 0, None) == -1
    assert lib.g4probe_mfma_bf16(FAKE, 1, 0, 0, None) == -1
    assert lib.g4probe_mfma_bf16(FAKE, 1, 1, 2, None) == -1
    assert lib.g4probe_mfma_bf16(FAKE, 1, 1, -1, None) == -1
    assert lib.g4probe_stream_read(None, 64, FAKE, 1, None) == -1
    assert lib.g4probe_stream_read(FAKE, 64, None, 1, None) == -1
    assert lib.g4probe_stream_read(ctypes.c_void_p(0x100008), 64, FAKE, 1, None) == -1
    assert lib.g4probe_stream_read(FAKE, 40, FAKE, 1, None) == -1
    assert lib.g4probe_stream_read(FAKE, 0, FAKE, 1, None) == -1
    assert lib.g4probe_stream_read(FAKE, 64, FAKE, 0, None) == -1


@pytest.mark.gpu
@pytest.mark.parametrize("n16,wgs", [(1, 1), (1000, 7), (300_001, 512)])
def test_stream_read_touches_every_element_once(n16, wgs):
    """The XOR of the sink equals the XOR of every word of the buffer: an element
    skipped or read twice (per workgroup chunk and tail) would change it."""
    import torch
    rng = np.random.default_rng(n16)
    words = rng.integers(0, 2 ** 32, size=4 * n16, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(words.view(np.int32)).cuda()
    sink = torch.full((wgs * 256,), -1, dtype=torch.int32, device="cuda")
    assert probe.stream_read(src, sink, wgs) == 16.0 * n16
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(words)


@pytest.mark.gpu
@pytest.mark.parametrize("operands", [probe.RANDOM, probe.LOW_ACTIVITY])
def test_mfma_loop_runs_every_round(operands):
    import torch
    wgs = 3
    out1 = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
    out3 = torch.empty_like(out1)
    assert probe.mfma_bf16(out1, wgs, 1, operands) == wgs * 4 * 1 * 8 * 32768
    probe.mfma_bf16(out3, wgs, 3, operands)
    torch.cuda.synchronize()
    assert torch.isfinite(out1).all() and out1.abs().sum() > 0
    torch.testing.assert_close(out3, 3.0 * out1, rtol=1e-5, atol=1e-4)
