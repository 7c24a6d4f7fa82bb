"""Build libjfa.so (the C-ABI library) in-tree with hipcc for gfx950.

Usage: ``python -m variable_length_flash_jagged_amd.build`` (or ``build()``).  Every
call recompiles all sources; objects go to ``_build/`` next to this file and the
library to ``libjfa.so`` in this package directory.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libjfa.so")

SOURCES = ["jfa_api.cpp", "jfa_sched.cpp", "jfa_fwd.hip", "jfa_bwd.hip", "jfa_bwd_self.hip", "jfa_bd.hip",
           "jfa_sparse.hip", "jfa_mxfp8.hip"]

# Packed fp32 VALU forms are disabled for all device code (the host pass warns that it
# does not know the feature; that warning is harmless).
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


# Per-source extra flags.  The dK/dV kernel runs at one wave per SIMD, where the
# compiler would otherwise put every MFMA result in accumulation registers and copy
# the scores out for the vector work (and the accumulators back and forth) on every
# step; the VGPR form keeps scores in VGPRs and uses the accumulation registers only
# for values that do not fit.
EXTRA_FLAGS = {"jfa_bwd_self.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [_hipcc()] + HIP_FLAGS + EXTRA_FLAGS.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if "not a recognized feature" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    return obj


def build(verbose=False, jobs=None):
    """Compile every source and link libjfa.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(8, len(SOURCES))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("linking libjfa.so failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
