"""Build libhmm.so (the HIP kernels and the C ABI) in-tree with hipcc for gfx950.

Usage: ``python -m mixture_experts_ffn_int32_amd.build`` (or ``build()``).
Every source is compiled for gfx950 only; packed-FP32 instructions are
disabled (``-packed-fp32-ops``).  Objects go to ``_build/`` and the library to
``mixture_experts_ffn_int32_amd/libhmm.so``.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libhmm.so")
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ["route.hip", "gemm.hip", "gemm_f32.hip", "gemm_fp8.hip", "quant.hip", "pointwise.hip", "fused.hip", "api.hip"]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libhmm)")


def flags(debug=False):
    f = ["-std=c++17", "--offload-arch=gfx950", "-fPIC", "-Wall", "-Wno-unused-result",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include")]
    f += ["-O1", "-g"] if debug else ["-O3"]
    return f


def _compile(src, obj, debug):
    cmd = [hipcc()] + flags(debug) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr[-8000:]))
    # keep real warnings visible, drop the host pass's note about the gfx-only feature flag
    warn = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
    return warn


def build(debug=False, verbose=True):
    """Compile every source and link libhmm.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = [os.path.join(BUILD_DIR, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        warns = list(ex.map(lambda so: _compile(so[0], so[1], debug), zip(SOURCES, objs)))
    for s, w in zip(SOURCES, warns):
        if w and verbose:
            print("[build] %s:\n%s" % (s, w), file=sys.stderr)
    tmp = OUT + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr[-8000:]))
    os.replace(tmp, OUT)
    if verbose:
        print("[build] wrote %s" % OUT, file=sys.stderr)
    return OUT


if __name__ == "__main__":
    build(debug="--debug" in sys.argv)
