"""Python binding of libg4attn: Gemma 4 decoder attention on MI355X (gfx950).

Argument marshalling only.  Every step of the computation runs in the HIP
kernels of ``libg4attn.so``; PyTorch supplies device memory and the current
stream.  If the library is missing, :func:`load` raises - there is no other
implementation to fall back on.

The functions carry the C names of ``include/g4attn.h``:

* :func:`g4attn_norm_rope` - RMSNorm (plain weight) + full / partial RoPE;
* :func:`g4attn_prefill`   - causal / sliding-window GQA attention, incl. K=V;
* :func:`g4attn_prefill_chunk` - the same for a chunk of new positions over caches;
* :func:`g4attn_decode`    - split-KV single-token decode over a KV cache.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libg4attn.so")

OK, ERR_NULL, ERR_SHAPE, ERR_LAYOUT, ERR_UNSUPPORTED, ERR_CACHE_OVERFLOW, ERR_WORKSPACE, ERR_HIP = range(8)

EXPORTED = ("g4attn_norm_rope", "g4attn_prefill_workspace_bytes", "g4attn_prefill", "g4attn_prefill_chunk",
            "g4attn_prefill_chunk_tied",
            "g4attn_decode_workspace_bytes", "g4attn_decode", "g4attn_decode_noalloc", "g4attn_kv_tied_append",
            "g4attn_decode_tied",
            "g4attn_status_str",
            "g4attn_last_hip_error", "g4attn_version")


class G4AttnError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = _lib.g4attn_status_str(status).decode() if _lib is not None else str(status)
        extra = ""
        if status == ERR_HIP and _lib is not None:
            extra = f" (hipError {_lib.g4attn_last_hip_error()})"
        super().__init__(f"{where}: {msg}{extra} [status {status}]")


class LayerDesc(ctypes.Structure):
    """Mirror of ``g4attn_layer_desc``."""
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("window", ctypes.c_int32),
                ("k_eq_v", ctypes.c_int32), ("rotary_dims", ctypes.c_int32),
                ("rope_theta", ctypes.c_float), ("rms_eps", ctypes.c_float),
                ("scale", ctypes.c_float)]


def layer_desc(num_q_heads, num_kv_heads, head_dim, window=0, k_eq_v=False, rotary_dims=None,
               rope_theta=1e6, rms_eps=1e-6, scale=None):
    if rotary_dims is None:
        rotary_dims = head_dim
    if scale is None:
        scale = head_dim ** -0.5
    return LayerDesc(num_q_heads, num_kv_heads, head_dim, window, int(bool(k_eq_v)), rotary_dims,
                     rope_theta, rms_eps, scale)


_lib = None
_P = ctypes.c_void_p
_I64x3 = ctypes.c_int64 * 3


def load(path=None):
    """Load libg4attn.so (once).  Raises if it has not been built.

    ``path`` or the environment variable ``G4ATTN_LIB`` selects another build
    of the same library.
    """
    global _lib
    if _lib is not None:
        return _lib
    path = path or os.environ.get("G4ATTN_LIB") or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"libg4attn.so not built ({path}); run "
                           "`python -m decoder_attention_g4attn_amd.build`")
    lib = ctypes.CDLL(path)
    lib.g4attn_norm_rope.restype = ctypes.c_int
    lib.g4attn_norm_rope.argtypes = [_P, _P, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_float,
                                     _P, _P, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P]
    lib.g4attn_prefill_workspace_bytes.restype = ctypes.c_size_t
    lib.g4attn_prefill_workspace_bytes.argtypes = [ctypes.POINTER(LayerDesc), ctypes.c_int32, ctypes.c_int32]
    lib.g4attn_prefill.restype = ctypes.c_int
    lib.g4attn_prefill.argtypes = [ctypes.POINTER(LayerDesc), _P, _P, _P, _P, _P, _P,
                                   ctypes.c_int32, ctypes.c_int32, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    lib.g4attn_prefill_chunk.restype = ctypes.c_int
    lib.g4attn_prefill_chunk.argtypes = [ctypes.POINTER(LayerDesc), _P, _P, _P, ctypes.c_int32, _P, _P,
                                         ctypes.c_int32, _P, _P, _P, _P, ctypes.c_int32, ctypes.c_int32, _P, _P, _P,
                                         ctypes.c_size_t, _P]
    lib.g4attn_prefill_chunk_tied.restype = ctypes.c_int
    lib.g4attn_prefill_chunk_tied.argtypes = [ctypes.POINTER(LayerDesc), _P, _P, _P, _P, _P, ctypes.c_int32, _P,
                                              _P, ctypes.c_int32, _P, _P, _P, _P, ctypes.c_int32, ctypes.c_int32,
                                              _P, _P, _P, ctypes.c_size_t, _P]
    lib.g4attn_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.g4attn_decode_workspace_bytes.argtypes = [ctypes.POINTER(LayerDesc), ctypes.c_int32,
                                                  ctypes.c_int32, ctypes.c_int32]
    lib.g4attn_decode.restype = ctypes.c_int
    lib.g4attn_decode.argtypes = [ctypes.POINTER(LayerDesc), _P, _P, _P, _P, ctypes.c_int32,
                                  ctypes.c_int32, ctypes.c_int32, _P, _P, ctypes.c_int32, _P,
                                  ctypes.c_size_t, _P]
    lib.g4attn_decode_noalloc.restype = ctypes.c_int
    lib.g4attn_decode_noalloc.argtypes = [ctypes.POINTER(LayerDesc), _P, _P, _P, _P, ctypes.c_int32,
                                          ctypes.c_int32, ctypes.c_int32, _P, _P, ctypes.c_int32, _P]
    lib.g4attn_kv_tied_append.restype = ctypes.c_int
    lib.g4attn_kv_tied_append.argtypes = [_P, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_float, ctypes.c_float, _P, _P, ctypes.c_int32, _P, _P, _P,
                                          ctypes.c_int32, _P]
    lib.g4attn_decode_tied.restype = ctypes.c_int
    lib.g4attn_decode_tied.argtypes = [ctypes.POINTER(LayerDesc), _P, _P, _P, _P, _P, _P, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_int32, _P, _P, ctypes.c_int32, _P, ctypes.c_size_t, _P]
    lib.g4attn_status_str.restype = ctypes.c_char_p
    lib.g4attn_status_str.argtypes = [ctypes.c_int]
    lib.g4attn_last_hip_error.restype = ctypes.c_int32
    lib.g4attn_last_hip_error.argtypes = []
    lib.g4attn_version.restype = ctypes.c_int32
    lib.g4attn_version.argtypes = []
    _lib = lib
    return lib


# ------------------------------------------------------------------ helpers
def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _bsh_strides(t):
    """(batch, seq, head) element strides of a [B, S, H, D] tensor with unit D stride."""
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("expected a [B, S, H, D] tensor with a unit D stride")
    return _I64x3(t.stride(0), t.stride(1), t.stride(2))


def _check_bf16(*ts):
    for t in ts:
        if t is not None and t.dtype != torch.bfloat16:
            raise TypeError("g4attn tensors are bfloat16")


def _expect(t, shape, name, dtype=None):
    """Raise unless ``t`` is a CUDA tensor of exactly ``shape`` (and ``dtype``)."""
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}")


def _raise(status, where):
    if status != OK:
        raise G4AttnError(status, where)


# --------------------------------------------------------------- entry points
def g4attn_norm_rope(x, y, weight, head_dim, rotary_dims, rope_theta, rms_eps=1e-6,
                     pos0=None, max_pos=None, cache_cap=0, ring=False, stream=None):
    """y = RoPE(RMSNorm(x) * weight) for x [B, S, H, D]; see g4attn_norm_rope in g4attn.h.

    ``cache_cap > 0``: ``y`` is a cache ``[B, H, cache_cap, D]`` written at rows
    ``pos0[b] + t`` (``ring``: at rows ``(pos0[b] + t) % cache_cap``, a sliding
    layer's rolling cache).  ``pos0`` is an int32 device tensor ``[B]`` or None.
    """
    lib = load()
    _check_bf16(x, y, weight)
    B, S, H, D = x.shape
    if D != head_dim:
        raise ValueError(f"x has head_dim {D}, expected {head_dim}")
    _expect(x, (B, S, H, D), "x")
    _expect(y, (B, H, cache_cap, D) if cache_cap else (B, S, H, D), "y")
    _expect(weight, (D,), "weight")
    _expect(pos0, (B,), "pos0", torch.int32)
    if cache_cap and not y.is_contiguous():
        raise ValueError("a cache must be contiguous")
    xs = _bsh_strides(x)
    ys = _I64x3(0, 0, 0) if cache_cap else _bsh_strides(y)
    if max_pos is None:
        max_pos = S - 1 if pos0 is None else int(pos0.max().item()) + S - 1
    st = lib.g4attn_norm_rope(_ptr(x), _ptr(y), _ptr(weight), B, S, H, head_dim, rotary_dims,
                              rope_theta, rms_eps, xs, ys, _ptr(pos0), max_pos, cache_cap, int(bool(ring)),
                              _stream(stream))
    _raise(st, "g4attn_norm_rope")
    return y


def g4attn_prefill_workspace_bytes(desc, B, S):
    return load().g4attn_prefill_workspace_bytes(ctypes.byref(desc), B, S)


def _spans(span_lo, span_hi):
    for t in (span_lo, span_hi):
        if t is not None and (t.dtype != torch.int32 or not t.is_contiguous()):
            raise TypeError("span bounds must be contiguous int32 [B, S]")
    return _ptr(span_lo), _ptr(span_hi)


def g4attn_prefill(desc, q, k, v, out, w_k=None, lse=None, workspace=None, stream=None, span_lo=None,
                   span_hi=None):
    """Prefill attention; see g4attn_prefill in g4attn.h.  Returns ``out``.

    For a K=V layer (``desc.k_eq_v``) pass the raw tied projection as ``k``,
    ``v=None`` and the K-norm weight as ``w_k``.  ``span_lo``/``span_hi``
    (int32 [B, S]) add bidirectional spans.  ``workspace`` (a uint8 device
    tensor) is allocated here if not given.
    """
    lib = load()
    _check_bf16(q, k, v, out, w_k)
    B, S = q.shape[0], q.shape[1]
    Hq, Hkv, D = desc.num_q_heads, desc.num_kv_heads, desc.head_dim
    _expect(q, (B, S, Hq, D), "q")
    _expect(k, (B, S, Hkv, D), "k")
    _expect(v, (B, S, Hkv, D), "v")
    _expect(out, (B, S, Hq, D), "out")
    _expect(w_k, (D,), "w_k")
    _expect(lse, (B, Hq, S), "lse", torch.float32)
    _expect(span_lo, (B, S), "span_lo")
    _expect(span_hi, (B, S), "span_hi")
    if lse is not None and not lse.is_contiguous():
        raise ValueError("lse must be contiguous")
    if v is not None and v.stride() != k.stride():
        raise ValueError("k and v must have the same strides (one kv_strides argument)")
    need = lib.g4attn_prefill_workspace_bytes(ctypes.byref(desc), B, S)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    lo, hi = _spans(span_lo, span_hi)
    st = lib.g4attn_prefill(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(w_k), _ptr(out),
                            _ptr(lse), B, S, _bsh_strides(q), _bsh_strides(k), _bsh_strides(out), lo, hi,
                            _ptr(workspace), wbytes, _stream(stream))
    _raise(st, "g4attn_prefill")
    return out


def g4attn_prefill_chunk(desc, q, k_cache, v_cache, out, pos0, qlen, max_pos=None, lse=None, workspace=None,
                         stream=None, span_lo=None, span_hi=None):
    """Chunked prefill over caches; see g4attn_prefill_chunk in g4attn.h.  Returns ``out``.

    ``q``/``out`` [B, S, Hq, D]; ``k_cache``, ``v_cache`` contiguous
    [B, Hkv, cap, D]; ``pos0``, ``qlen`` int32 device tensors [B].
    ``max_pos`` (the bound of every pos0[b] + qlen[b] - 1) is read from
    ``pos0`` and ``qlen`` when not given (a device-to-host copy).
    """
    lib = load()
    _check_bf16(q, k_cache, v_cache, out)
    B, S = q.shape[0], q.shape[1]
    Hq, Hkv, D = desc.num_q_heads, desc.num_kv_heads, desc.head_dim
    cap = k_cache.shape[2]
    _expect(q, (B, S, Hq, D), "q")
    _expect(out, (B, S, Hq, D), "out")
    _expect(k_cache, (B, Hkv, cap, D), "k_cache")
    _expect(v_cache, (B, Hkv, cap, D), "v_cache")
    _expect(pos0, (B,), "pos0", torch.int32)
    _expect(qlen, (B,), "qlen", torch.int32)
    _expect(lse, (B, Hq, S), "lse", torch.float32)
    _expect(span_lo, (B, S), "span_lo")
    _expect(span_hi, (B, S), "span_hi")
    for t in (k_cache, v_cache):
        if not t.is_contiguous():
            raise ValueError("caches must be contiguous")
    if max_pos is None:
        max_pos = int((pos0.to(torch.int64) + qlen.to(torch.int64)).max().item()) - 1
    need = lib.g4attn_prefill_workspace_bytes(ctypes.byref(desc), B, S)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wbytes = workspace.numel() * workspace.element_size()
    lo, hi = _spans(span_lo, span_hi)
    st = lib.g4attn_prefill_chunk(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache), k_cache.shape[2],
                                  _ptr(pos0), _ptr(qlen), max_pos, lo, hi, _ptr(out), _ptr(lse), B, S,
                                  _bsh_strides(q), _bsh_strides(out), _ptr(workspace), wbytes, _stream(stream))
    _raise(st, "g4attn_prefill_chunk")
    return out


def g4attn_prefill_chunk_tied(desc, q, x_cache, r_cache, krot_cache, w_k, out, pos0, qlen, max_pos=None, lse=None,
                              workspace=None, stream=None, span_lo=None, span_hi=None):
    """Chunked prefill of a K=V layer over its raw-projection cache; see
    g4attn_prefill_chunk_tied in g4attn.h.  Returns ``out``.

    ``q``/``out`` [B, S, Hq, 512]; ``x_cache`` [B, Hkv, cap, 512], ``r_cache``
    fp32 [B, Hkv, cap], ``krot_cache`` [B, Hkv, cap, 128] (as
    g4attn_kv_tied_append writes them), all contiguous; ``pos0``, ``qlen``
    int32 device tensors [B]; ``max_pos`` as in :func:`g4attn_prefill_chunk`.
    """
    lib = load()
    _check_bf16(q, x_cache, krot_cache, w_k, out)
    B, S = q.shape[0], q.shape[1]
    Hq, Hkv, D = desc.num_q_heads, desc.num_kv_heads, desc.head_dim
    cap = x_cache.shape[2]
    _expect(q, (B, S, Hq, D), "q")
    _expect(out, (B, S, Hq, D), "out")
    _expect(x_cache, (B, Hkv, cap, D), "x_cache")
    _expect(r_cache, (B, Hkv, cap), "r_cache", torch.float32)
    _expect(krot_cache, (B, Hkv, cap, 128), "krot_cache")
    _expect(w_k, (D,), "w_k")
    _expect(pos0, (B,), "pos0", torch.int32)
    _expect(qlen, (B,), "qlen", torch.int32)
    _expect(lse, (B, Hq, S), "lse", torch.float32)
    _expect(span_lo, (B, S), "span_lo")
    _expect(span_hi, (B, S), "span_hi")
    for t in (x_cache, r_cache, krot_cache, w_k):
        if not t.is_contiguous():
            raise ValueError("caches and w_k must be contiguous")
    if max_pos is None:
        max_pos = int((pos0.to(torch.int64) + qlen.to(torch.int64)).max().item()) - 1
    need = lib.g4attn_prefill_workspace_bytes(ctypes.byref(desc), B, S)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wbytes = workspace.numel() * workspace.element_size()
    lo, hi = _spans(span_lo, span_hi)
    st = lib.g4attn_prefill_chunk_tied(ctypes.byref(desc), _ptr(q), _ptr(x_cache), _ptr(r_cache),
                                       _ptr(krot_cache), _ptr(w_k), cap, _ptr(pos0), _ptr(qlen), max_pos, lo, hi,
                                       _ptr(out), _ptr(lse), B, S, _bsh_strides(q), _bsh_strides(out),
                                       _ptr(workspace), wbytes, _stream(stream))
    _raise(st, "g4attn_prefill_chunk_tied")
    return out


def g4attn_decode_workspace_bytes(desc, B, max_kv_len, num_splits=0):
    return load().g4attn_decode_workspace_bytes(ctypes.byref(desc), B, max_kv_len, num_splits)


def g4attn_decode(desc, q, k_cache, v_cache, kv_len, max_kv_len, out, lse=None, num_splits=0,
                  workspace=None, stream=None):
    """Split-KV decode; see g4attn_decode in g4attn.h.  Returns ``out``.

    ``q`` [B, Hq, D], caches [B, Hkv, cap, D] (``v_cache`` may be ``k_cache``),
    ``kv_len`` int32 device tensor [B].  Sliding layers (``desc.window > 0``)
    read a ring cache of ``cap == window`` slots (see g4attn_norm_rope's ring).
    """
    lib = load()
    _check_bf16(q, k_cache, v_cache, out)
    if kv_len.dtype != torch.int32:
        raise TypeError("kv_len must be int32")
    for t in (q, k_cache, v_cache, out):
        if not t.is_contiguous():
            raise ValueError("decode tensors must be contiguous")
    B = q.shape[0]
    cap = k_cache.shape[2]
    Hq, Hkv, D = desc.num_q_heads, desc.num_kv_heads, desc.head_dim
    _expect(q, (B, Hq, D), "q")
    _expect(out, (B, Hq, D), "out")
    _expect(k_cache, (B, Hkv, cap, D), "k_cache")
    _expect(v_cache, (B, Hkv, cap, D), "v_cache")
    _expect(kv_len, (B,), "kv_len", torch.int32)
    _expect(lse, (B, Hq), "lse", torch.float32)
    need = lib.g4attn_decode_workspace_bytes(ctypes.byref(desc), B, max_kv_len, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    wbytes = workspace.numel() * workspace.element_size()
    st = lib.g4attn_decode(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(kv_len),
                           B, max_kv_len, cap, _ptr(out), _ptr(lse), num_splits, _ptr(workspace),
                           wbytes, _stream(stream))
    _raise(st, "g4attn_decode")
    return out


def g4attn_decode_noalloc(desc, q, k_cache, v_cache, kv_len, max_kv_len, out, lse=None, num_splits=0,
                          stream=None):
    """g4attn_decode without a workspace (the library's own per-GPU scratch
    array); see g4attn_decode_noalloc in g4attn.h.  Allocates nothing.  Returns ``out``."""
    lib = load()
    _check_bf16(q, k_cache, v_cache, out)
    for t in (q, k_cache, v_cache, out):
        if not t.is_contiguous():
            raise ValueError("decode tensors must be contiguous")
    B = q.shape[0]
    cap = k_cache.shape[2]
    Hq, Hkv, D = desc.num_q_heads, desc.num_kv_heads, desc.head_dim
    _expect(q, (B, Hq, D), "q")
    _expect(out, (B, Hq, D), "out")
    _expect(k_cache, (B, Hkv, cap, D), "k_cache")
    _expect(v_cache, (B, Hkv, cap, D), "v_cache")
    _expect(kv_len, (B,), "kv_len", torch.int32)
    _expect(lse, (B, Hq), "lse", torch.float32)
    st = lib.g4attn_decode_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(kv_len),
                                   B, max_kv_len, cap, _ptr(out), _ptr(lse), num_splits, _stream(stream))
    _raise(st, "g4attn_decode_noalloc")
    return out


def g4attn_kv_tied_append(x, w_k, x_cache, r_cache, krot_cache, rope_theta, rms_eps=1e-6, pos0=None,
                          max_pos=None, rotary_dims=128, stream=None):
    """Append raw K=V rows X [B, S, Hkv, 512] to a K=V cache; see g4attn_kv_tied_append."""
    lib = load()
    _check_bf16(x, w_k, x_cache, krot_cache)
    if r_cache.dtype != torch.float32:
        raise TypeError("r_cache is float32")
    for t in (x_cache, r_cache, krot_cache):
        if not t.is_contiguous():
            raise ValueError("caches must be contiguous")
    B, S, Hkv, D = x.shape
    cap = x_cache.shape[2]
    _expect(x, (B, S, Hkv, 512), "x")
    _expect(w_k, (512,), "w_k")
    _expect(x_cache, (B, Hkv, cap, 512), "x_cache")
    _expect(r_cache, (B, Hkv, cap), "r_cache")
    _expect(krot_cache, (B, Hkv, cap, 128), "krot_cache")
    _expect(pos0, (B,), "pos0", torch.int32)
    if max_pos is None:
        max_pos = S - 1 if pos0 is None else int(pos0.max().item()) + S - 1
    st = lib.g4attn_kv_tied_append(_ptr(x), _ptr(w_k), B, S, Hkv, rotary_dims, rope_theta, rms_eps,
                                   _bsh_strides(x), _ptr(pos0), max_pos, _ptr(x_cache), _ptr(r_cache),
                                   _ptr(krot_cache), x_cache.shape[2], _stream(stream))
    _raise(st, "g4attn_kv_tied_append")


def g4attn_decode_tied(desc, q, x_cache, r_cache, krot_cache, w_k, kv_len, max_kv_len, out, lse=None,
                       num_splits=0, workspace=None, stream=None):
    """K=V decode over the raw-projection cache; see g4attn_decode_tied in g4attn.h.  Returns ``out``."""
    lib = load()
    _check_bf16(q, x_cache, krot_cache, w_k, out)
    if kv_len.dtype != torch.int32:
        raise TypeError("kv_len must be int32")
    for t in (q, x_cache, r_cache, krot_cache, out):
        if not t.is_contiguous():
            raise ValueError("decode tensors must be contiguous")
    B = q.shape[0]
    Hq, Hkv, D = desc.num_q_heads, desc.num_kv_heads, desc.head_dim
    cap = x_cache.shape[2]
    _expect(q, (B, Hq, D), "q")
    _expect(out, (B, Hq, D), "out")
    _expect(x_cache, (B, Hkv, cap, D), "x_cache")
    _expect(r_cache, (B, Hkv, cap), "r_cache", torch.float32)
    _expect(krot_cache, (B, Hkv, cap, 128), "krot_cache")
    _expect(w_k, (D,), "w_k")
    _expect(kv_len, (B,), "kv_len", torch.int32)
    _expect(lse, (B, Hq), "lse", torch.float32)
    need = lib.g4attn_decode_workspace_bytes(ctypes.byref(desc), B, max_kv_len, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    wbytes = workspace.numel() * workspace.element_size()
    st = lib.g4attn_decode_tied(ctypes.byref(desc), _ptr(q), _ptr(x_cache), _ptr(r_cache), _ptr(krot_cache),
                                _ptr(w_k), _ptr(kv_len), B, max_kv_len, x_cache.shape[2], _ptr(out), _ptr(lse),
                                num_splits, _ptr(workspace), wbytes, _stream(stream))
    _raise(st, "g4attn_decode_tied")
    return out


def g4attn_status_str(status):
    return load().g4attn_status_str(status).decode()


def g4attn_version():
    return load().g4attn_version()
