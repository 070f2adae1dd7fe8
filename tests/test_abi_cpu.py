"""The C ABI without a GPU: the library loads, exports every declared symbol,
and rejects invalid calls on the host before any HIP call (no compute)."""

import ctypes
import os
import re

import pytest

import decoder_attention_g4attn_amd as g4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "g4attn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(g4.LIB_PATH), reason="libg4attn.so not built")

FAKE = ctypes.c_void_p(0x100000)      # 16-byte aligned, never dereferenced
MISALIGNED = ctypes.c_void_p(0x100008)
I64 = ctypes.c_int64 * 3


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\S.*?\b(g4attn_\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol():
    lib = g4.load()
    decl = declared_functions()
    assert set(decl) == set(g4.EXPORTED)
    for name in decl:
        assert hasattr(lib, name), name


def test_header_serves_a_plain_c_caller(tmp_path):
    """The header is plain C99 (no C++ types leak into the signatures) and a C program links
    against the library and gets a host-side validation error back without any GPU."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "caller.c"
    src.write_text(
        "#include <stdio.h>\n#include \"g4attn.h\"\n"
        "int main(void) {\n"
        "  g4attn_status s = g4attn_prefill(NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1, 1, NULL, NULL, NULL,\n"
        "                                   NULL, NULL, NULL, 0, NULL);\n"
        "  printf(\"%d %d %s\\n\", (int)g4attn_version(), (int)s, g4attn_status_str(s));\n"
        "  return s == G4ATTN_ERR_NULL ? 0 : 1;\n}\n")
    exe = tmp_path / "caller"
    libdir = os.path.dirname(g4.LIB_PATH)
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", os.path.dirname(HEADER),
                        str(src), "-o", str(exe), "-L", libdir, "-lg4attn", f"-Wl,-rpath,{libdir}"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    version, status, text = r.stdout.split(" ", 2)
    assert int(version) == g4.load().g4attn_version() and int(status) == 1 and "NULL" in text


def test_version_and_status_strings():
    assert g4.g4attn_version() == 400
    for s in range(8):
        assert g4.g4attn_status_str(s)
    assert g4.load().g4attn_last_hip_error() == 0


def _desc(**kw):
    d = dict(num_q_heads=32, num_kv_heads=4, head_dim=512, window=0, k_eq_v=False,
             rotary_dims=128, rope_theta=1e6)
    d.update(kw)
    return g4.layer_desc(**d)


def _prefill(desc, q=FAKE, k=FAKE, v=FAKE, wk=None, out=FAKE, B=1, S=16, qs=None, ks=None, os_=None,
             ws=None, wsb=0, span_lo=None, span_hi=None):
    lib = g4.load()
    qs = qs or I64(16 * 32 * 512, 32 * 512, 512)
    ks = ks or I64(16 * 4 * 512, 4 * 512, 512)
    os_ = os_ or I64(16 * 32 * 512, 32 * 512, 512)
    return lib.g4attn_prefill(ctypes.byref(desc), q, k, v, wk, out, None, B, S, qs, ks, os_, span_lo, span_hi,
                              ws, wsb, None)


def test_prefill_validation():
    assert _prefill(_desc(), q=None) == g4.ERR_NULL
    assert _prefill(_desc(), v=None) == g4.ERR_NULL
    assert _prefill(_desc(num_q_heads=30)) == g4.ERR_SHAPE            # Hq % Hkv
    assert _prefill(_desc(head_dim=128, rotary_dims=128)) == g4.ERR_UNSUPPORTED
    assert _prefill(_desc(rotary_dims=100)) == g4.ERR_UNSUPPORTED
    assert _prefill(_desc(window=-1)) == g4.ERR_SHAPE
    assert _prefill(_desc(), S=0) == g4.ERR_SHAPE
    assert _prefill(_desc(), B=0) == g4.ERR_SHAPE
    assert _prefill(_desc(), q=MISALIGNED) == g4.ERR_LAYOUT
    assert _prefill(_desc(), qs=I64(16 * 32 * 512, 32 * 512, 511)) == g4.ERR_LAYOUT
    # K/V row strides of 2^25 elements or more: tile row offsets would overflow 32 bits
    assert _prefill(_desc(), ks=I64(16 * (1 << 25), 1 << 25, 512), ws=FAKE, wsb=1 << 30) == g4.ERR_UNSUPPORTED
    # K=V layer: one tensor, K weight required, D = 512 with 128 rotated dims
    kv = _desc(k_eq_v=True)
    assert _prefill(kv, wk=None, v=None) == g4.ERR_NULL
    assert _prefill(kv, wk=FAKE, v=FAKE) == g4.ERR_SHAPE
    assert _prefill(_desc(k_eq_v=True, rotary_dims=512), wk=FAKE, v=None) == g4.ERR_UNSUPPORTED
    assert _prefill(_desc(k_eq_v=True, scale=2.0 ** 31), wk=FAKE, v=None) == g4.ERR_UNSUPPORTED
    need = g4.g4attn_prefill_workspace_bytes(kv, 1, 16)
    # flags [1, 4, 1 tile, 4 waves] + r [1, 4, 16] + Krot [1, 4, 16, 128], each 256-byte aligned
    assert need == 256 + 256 + 16 * 4 * 128 * 2
    assert _prefill(kv, wk=FAKE, v=None) == g4.ERR_WORKSPACE
    # bidirectional spans: both bounds or neither; K=V layers take them too
    assert _prefill(_desc(), span_lo=FAKE) == g4.ERR_NULL
    assert _prefill(kv, wk=FAKE, v=None, span_lo=FAKE, span_hi=FAKE) == g4.ERR_WORKSPACE
    assert _prefill(kv, wk=FAKE, v=None, ws=FAKE, wsb=need - 1) == g4.ERR_WORKSPACE
    assert g4.g4attn_prefill_workspace_bytes(_desc(), 1, 16) == 256
    assert _prefill(_desc()) == g4.ERR_WORKSPACE


def _decode(desc, B=2, max_len=100, cap=128, splits=0, ws=FAKE, wsb=1 << 30, q=FAKE, kc=FAKE, kl=FAKE):
    lib = g4.load()
    return lib.g4attn_decode(ctypes.byref(desc), q, kc, kc, kl, B, max_len, cap, FAKE, None, splits,
                             ws, wsb, None)


def test_decode_validation():
    assert _decode(_desc(), q=None) == g4.ERR_NULL
    assert _decode(_desc(), kl=None) == g4.ERR_NULL
    assert _decode(_desc(), max_len=129, cap=128) == g4.ERR_CACHE_OVERFLOW    # cache overflow raises
    # sliding layer: the cache must be a ring of exactly `window` slots
    assert _decode(_desc(window=1024)) == g4.ERR_SHAPE
    assert _decode(_desc(num_q_heads=64, num_kv_heads=2)) == g4.ERR_UNSUPPORTED   # > 16 heads per group
    assert _decode(_desc(), max_len=0) == g4.ERR_SHAPE
    assert _decode(_desc(), splits=-1) == g4.ERR_SHAPE
    assert _decode(_desc(), wsb=16) == g4.ERR_WORKSPACE
    assert _decode(_desc(), ws=None) == g4.ERR_WORKSPACE
    assert _decode(_desc(), kc=MISALIGNED) == g4.ERR_LAYOUT


def test_decode_workspace_sizes():
    d = _desc()
    # automatic chunking: >= 256 rows, multiple of 64
    ws = g4.g4attn_decode_workspace_bytes(d, 32, 131073, 0)
    assert ws > 0
    for splits in (1, 2, 7):
        w = g4.g4attn_decode_workspace_bytes(d, 2, 1000, splits)
        chunk = -(-(-(-1000 // splits)) // 64) * 64
        ns = -(-1000 // chunk)
        a256 = lambda x: -(-x // 256) * 256
        assert w == a256(2 * 32 * ns * 512 * 4) + 2 * a256(2 * 32 * ns * 4) + a256(2 * 4 * ns * 4)


def test_prefill_chunk_validation():
    lib = g4.load()
    qs = I64(16 * 32 * 256, 32 * 256, 256)

    def call(desc=None, q=FAKE, kc=FAKE, vc=FAKE, cap=64, pos0=FAKE, qlen=FAKE, max_pos=40, B=1, S=16,
             ws=None, wsb=0):
        desc = desc or _desc(head_dim=256, rotary_dims=256)
        return lib.g4attn_prefill_chunk(ctypes.byref(desc), q, kc, vc, cap, pos0, qlen, max_pos, None, None, FAKE,
                                        None, B, S, qs, qs, ws, wsb, None)

    assert call(pos0=None) == g4.ERR_NULL
    assert call(qlen=None) == g4.ERR_NULL
    assert call(desc=_desc(k_eq_v=True), ws=FAKE, wsb=1 << 30) == g4.ERR_UNSUPPORTED
    assert call(max_pos=64) == g4.ERR_CACHE_OVERFLOW     # the last position must fit the cache
    assert call(max_pos=-1) == g4.ERR_SHAPE
    assert call(S=0) == g4.ERR_SHAPE
    assert call(q=MISALIGNED) == g4.ERR_LAYOUT
    assert call() == g4.ERR_WORKSPACE


def test_kv_tied_cache_validation():
    lib = g4.load()
    xs = I64(16 * 4 * 512, 4 * 512, 512)

    def append(x=FAKE, wk=FAKE, rot=128, pos0=None, max_pos=15, cap=64, S=16):
        return lib.g4attn_kv_tied_append(x, wk, 1, S, 4, rot, 1e6, 1e-6, xs, pos0, max_pos, FAKE, FAKE, FAKE,
                                         cap, None)

    assert append(wk=None) == g4.ERR_NULL
    assert append(rot=256) == g4.ERR_UNSUPPORTED
    assert append(cap=15) == g4.ERR_CACHE_OVERFLOW
    assert append(pos0=FAKE, max_pos=10) == g4.ERR_SHAPE
    assert append(x=MISALIGNED) == g4.ERR_LAYOUT

    def decode(desc, max_len=100, cap=128, ws=FAKE, wsb=1 << 30, wk=FAKE):
        return lib.g4attn_decode_tied(ctypes.byref(desc), FAKE, FAKE, FAKE, FAKE, wk, FAKE, 2, max_len, cap, FAKE,
                                      None, 0, ws, wsb, None)

    kv = _desc(k_eq_v=True)
    assert decode(kv, wk=None) == g4.ERR_NULL
    assert decode(_desc()) == g4.ERR_UNSUPPORTED                      # not a K=V layer
    assert decode(_desc(k_eq_v=True, window=16)) == g4.ERR_UNSUPPORTED
    assert decode(kv, max_len=200) == g4.ERR_CACHE_OVERFLOW
    assert decode(kv, ws=None) == g4.ERR_WORKSPACE


def test_decode_ring_workspace_uses_window_rows():
    """A sliding layer's decode reads at most `window` rows of its ring, however long the sequence."""
    ring = _desc(num_q_heads=32, num_kv_heads=16, head_dim=256, window=1024, rotary_dims=256)
    glob = _desc(num_q_heads=32, num_kv_heads=16, head_dim=256, window=0, rotary_dims=256)
    assert g4.g4attn_decode_workspace_bytes(ring, 32, 131073, 0) == g4.g4attn_decode_workspace_bytes(glob, 32, 1024, 0)
    assert g4.g4attn_decode_workspace_bytes(ring, 32, 700, 3) == g4.g4attn_decode_workspace_bytes(glob, 32, 700, 3)


def test_norm_rope_validation():
    lib = g4.load()
    xs = I64(16 * 8 * 256, 8 * 256, 256)

    def call(x=FAKE, y=FAKE, B=1, S=16, H=8, D=256, rot=256, theta=1e4, pos0=None, max_pos=15, cap=0,
             strides=xs, ring=0):
        return lib.g4attn_norm_rope(x, y, None, B, S, H, D, rot, theta, 1e-6, strides, strides, pos0,
                                    max_pos, cap, ring, None)

    assert call(x=None) == g4.ERR_NULL
    assert call(S=0) == g4.ERR_SHAPE
    assert call(D=128, rot=128) == g4.ERR_UNSUPPORTED
    assert call(rot=96) == g4.ERR_UNSUPPORTED
    assert call(theta=0.0) == g4.ERR_SHAPE
    assert call(x=MISALIGNED) == g4.ERR_LAYOUT
    assert call(strides=I64(16 * 8 * 256, 8 * 256, 255)) == g4.ERR_LAYOUT
    # cache mode: the last written row must fit
    assert call(cap=15) == g4.ERR_CACHE_OVERFLOW
    assert call(pos0=FAKE, max_pos=40, cap=40) == g4.ERR_CACHE_OVERFLOW
    assert call(pos0=FAKE, max_pos=10) == g4.ERR_SHAPE     # max_pos < S - 1
    # ring mode needs a cache and is a flag
    assert call(ring=1) == g4.ERR_SHAPE
    assert call(cap=64, ring=2) == g4.ERR_SHAPE


def test_decode_noalloc_validation():
    """The no-workspace decode validates like g4attn_decode, before any HIP call."""
    lib = g4.load()
    d = _desc()

    def call(q=FAKE, k=FAKE, v=FAKE, kv_len=FAKE, B=2, max_len=100, cap=128, out=FAKE, splits=0, desc=d):
        return lib.g4attn_decode_noalloc(ctypes.byref(desc), q, k, v, kv_len, B, max_len, cap, out, None,
                                         splits, None)
    assert call(q=None) == g4.ERR_NULL
    assert call(kv_len=None) == g4.ERR_NULL
    assert call(B=0) == g4.ERR_SHAPE
    assert call(max_len=200) == g4.ERR_CACHE_OVERFLOW
    assert call(out=MISALIGNED) == g4.ERR_LAYOUT
    assert call(desc=_desc(num_q_heads=30)) == g4.ERR_SHAPE
    # partial results beyond the 32 MiB scratch array, even as one split
    assert call(B=4096, max_len=64, cap=64) == g4.ERR_WORKSPACE
    # an explicit split count whose partial results do not fit
    assert call(B=64, max_len=100000, cap=100000, splits=64) == g4.ERR_WORKSPACE


def test_prefill_chunk_tied_validation():
    lib = g4.load()
    qs = I64(16 * 32 * 512, 32 * 512, 512)
    kv = _desc(k_eq_v=True)

    def call(desc=kv, q=FAKE, xc=FAKE, rc=FAKE, kr=FAKE, wk=FAKE, cap=64, pos0=FAKE, qlen=FAKE, max_pos=40, B=1,
             S=16, ws=None, wsb=0, lo=None, hi=None):
        return lib.g4attn_prefill_chunk_tied(ctypes.byref(desc), q, xc, rc, kr, wk, cap, pos0, qlen, max_pos, lo,
                                             hi, FAKE, None, B, S, qs, qs, ws, wsb, None)

    assert call(xc=None) == g4.ERR_NULL
    assert call(rc=None) == g4.ERR_NULL
    assert call(kr=None) == g4.ERR_NULL
    assert call(wk=None) == g4.ERR_NULL
    assert call(pos0=None) == g4.ERR_NULL
    assert call(lo=FAKE) == g4.ERR_NULL                                    # spans come as a pair
    assert call(desc=_desc()) == g4.ERR_UNSUPPORTED                       # not a K=V layer
    assert call(desc=_desc(k_eq_v=True, rotary_dims=512)) == g4.ERR_UNSUPPORTED
    assert call(desc=_desc(k_eq_v=True, scale=2.0 ** 31)) == g4.ERR_UNSUPPORTED
    assert call(max_pos=64) == g4.ERR_CACHE_OVERFLOW
    assert call(B=0) == g4.ERR_SHAPE
    assert call(rc=ctypes.c_void_p(0x100002), ws=FAKE, wsb=1 << 30) == g4.ERR_LAYOUT        # r cache not 4-byte aligned
    assert call(xc=MISALIGNED, ws=FAKE, wsb=1 << 30) == g4.ERR_LAYOUT
    # only the flags are needed: [1, 4, 1 tile, 4 waves] ints, 256-byte aligned
    assert call(ws=FAKE, wsb=255) == g4.ERR_WORKSPACE


def test_binding_checks_tensors_before_calling_the_library():
    """The binding refuses host tensors, wrong dtypes and wrong shapes itself (the C ABI sees only
    pointers), before any library call."""
    import torch
    desc = _desc(head_dim=256, rotary_dims=256)
    q = torch.zeros((1, 4, 32, 256), dtype=torch.bfloat16)
    kv = torch.zeros((1, 4, 4, 256), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device tensor"):
        g4.g4attn_prefill(desc, q, kv, kv, torch.empty_like(q))
    with pytest.raises(TypeError):
        g4.g4attn_prefill(desc, q.float(), kv, kv, q)

    class Dev:  # a stand-in with the attributes the shape check reads
        is_cuda = True

        def __init__(self, shape, dtype=torch.bfloat16):
            self.shape, self.dtype = shape, dtype

    g4._expect(Dev((1, 4, 32, 256)), (1, 4, 32, 256), "q")
    g4._expect(None, (1,), "optional")
    with pytest.raises(ValueError, match="shape"):
        g4._expect(Dev((1, 4, 16, 256)), (1, 4, 32, 256), "q")
    with pytest.raises(TypeError):
        g4._expect(Dev((2,), torch.int64), (2,), "pos0", torch.int32)
