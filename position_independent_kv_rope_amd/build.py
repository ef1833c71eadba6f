"""Build libpic.so (the C-ABI library) in-tree with hipcc for gfx950.

Usage: python -m position_independent_kv_rope_amd.build   (or call build()).
"""

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpic.so")
# calibration kernels for the measured peaks bench.py reports (include/pic_calib.h)
CALIB_LIB = os.path.join(PKG, "libpic_calib.so")
CALIB_SOURCES = ["pic_calib.hip"]

SOURCES = ["pic_plan.cpp", "pic_rope_splice.hip", "pic_attn.hip", "pic_attn_paged.hip",
           "pic_decode.hip", "pic_link.hip", "pic_state.hip"]

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU instructions.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; ROCm is required to build libpic.so")


def _link(sources, lib, verbose):
    srcs = [os.path.join(CSRC, s) for s in sources]
    tmp = lib + ".tmp"
    cmd = [hipcc()] + FLAGS + ["-I", INCLUDE, "-I", CSRC, "-o", tmp] + srcs
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = [ln for ln in res.stderr.splitlines() if "is not a recognized feature" not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed (%d):\n%s" % (res.returncode, "\n".join(errs)))
    if verbose and errs:
        print("\n".join(errs), file=sys.stderr)
    os.replace(tmp, lib)


def build(verbose=False):
    """Compile every source into libpic.so, and the calibration kernels into
    libpic_calib.so (always recompiles)."""
    _link(SOURCES, LIB, verbose)
    _link(CALIB_SOURCES, CALIB_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
