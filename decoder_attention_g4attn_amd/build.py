"""Build libg4attn.so and libg4probe.so in-tree with hipcc for gfx950.

    python -m decoder_attention_g4attn_amd.build [-v]

Every HIP source under csrc/ is compiled to an object in _build/ and linked
into ``decoder_attention_g4attn_amd/libg4attn.so``; the roofline probes under
probes/ go into ``decoder_attention_g4attn_amd/libg4probe.so``.  Always
recompiles.
"""

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libg4attn.so")
PROBES = os.path.join(PKG, "probes")
PROBE_LIB = os.path.join(PKG, "libg4probe.so")
ARCH = "gfx950"

CXXFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from forming packed fp32 VALU ops on the device
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
    "-I", os.path.join(ROOT, "include"),
]


# Per-source extra flags.  prefill.hip: MFMA builtins write VGPRs (the score
# tile), because its O accumulator lives in AGPRs via inline assembly.
EXTRA = {"prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [_hipcc(), *CXXFLAGS, *EXTRA.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    if verbose and msgs.strip():
        print(msgs)
    return obj


def _link(objs, lib, verbose):
    tmp = lib + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, lib)
    if verbose:
        print("built", lib)


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    probe_srcs = sorted(os.path.join(PROBES, f) for f in os.listdir(PROBES) if f.endswith(".hip"))
    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), sources() + probe_srcs))
    n = len(objs) - len(probe_srcs)
    _link(objs[:n], LIB, verbose)
    _link(objs[n:], PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
