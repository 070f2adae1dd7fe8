"""ctypes binding of libg4probe.so: the roofline probes declared in
include/g4probe.h (a bare bf16 MFMA loop and an HBM streaming read).

Argument marshalling only; the work runs in the library's kernels.  Tensors
are torch CUDA tensors, launched on torch's current stream.
"""

import ctypes
import os

PROBE_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libg4probe.so")
_lib = None
RANDOM, LOW_ACTIVITY = 0, 1  # operand data of the MFMA loop (G4PROBE_RANDOM, G4PROBE_LOW_ACTIVITY)


def load(path=None):
    """Load libg4probe.so (``path``, else ``G4PROBE_LIB``, else the in-tree build)."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or os.environ.get("G4PROBE_LIB") or PROBE_LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run python -m decoder_attention_g4attn_amd.build")
    lib = ctypes.CDLL(path)
    lib.g4probe_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                      ctypes.c_void_p]
    lib.g4probe_mfma_bf16.restype = ctypes.c_int
    lib.g4probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32,
                                        ctypes.c_void_p]
    lib.g4probe_stream_read.restype = ctypes.c_int
    _lib = lib
    return lib


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(rc, name):
    if rc != 0:
        raise RuntimeError(f"{name} failed with code {rc}")


def mfma_bf16(out, workgroups, iters, operands=RANDOM):
    """Launch the MFMA loop; ``out`` is a float32 CUDA tensor of >= workgroups*256 elements.
    Returns the flop count of the launch."""
    import torch
    if out.dtype != torch.float32 or not out.is_cuda or out.numel() < workgroups * 256:
        raise ValueError("out must be a float32 CUDA tensor of workgroups*256 elements")
    _check(load().g4probe_mfma_bf16(ctypes.c_void_p(out.data_ptr()), workgroups, iters, operands, _stream()),
           "g4probe_mfma_bf16")
    return float(workgroups) * 4 * iters * 8 * 32768


def stream_read(src, sink, workgroups):
    """Launch the streaming read over every byte of ``src`` (a contiguous CUDA tensor);
    ``sink`` is an int32/uint32-sized CUDA tensor of >= workgroups*256 elements.
    Returns the bytes read."""
    if not src.is_cuda or not src.is_contiguous() or not sink.is_cuda or sink.element_size() != 4 \
            or sink.numel() < workgroups * 256:
        raise ValueError("src must be a contiguous CUDA tensor and sink a 4-byte CUDA tensor of workgroups*256")
    nbytes = src.numel() * src.element_size()
    _check(load().g4probe_stream_read(ctypes.c_void_p(src.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()),
                                      workgroups, _stream()), "g4probe_stream_read")
    return float(nbytes)
