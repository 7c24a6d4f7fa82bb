"""Build libjfa.so (the C-ABI library) in-tree with hipcc for gfx950.

Usage: ``python -m variable_length_flash_jagged_amd.build`` (or ``build()``).  Every
call recompiles all sources; objects go to ``_build/`` next to this file and the
library to ``libjfa.so`` in this package directory.

``python -m variable_length_flash_jagged_amd.build --resource-usage OUT.md`` instead
compiles every device source once more with the compiler's kernel resource remarks and
writes, per kernel, its registers (VGPR, AGPR, SGPR), spills, scratch, LDS and
occupancy as a Markdown table (no library is linked).
"""

import concurrent.futures
import os
import re
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
           "jfa_sparse.hip", "jfa_mxfp8.hip", "jfa_noalloc.hip"]

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
# for values that do not fit.  The atomic optimizer is off there: its rewrite of the
# single-lane tile reservation reads the result at once (a vmcnt(0) wait that also waits
# for every copy in flight), where the kernels consume it a whole tile later.
EXTRA_FLAGS = {"jfa_bwd_self.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]}


def _hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src, verbose, extra=(), obj=None):
    obj = obj or os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [_hipcc()] + HIP_FLAGS + EXTRA_FLAGS.get(src, []) + list(extra) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if "not a recognized feature" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    return msgs if extra else obj


_FIELDS = [("VGPRs", "VGPR"), ("AGPRs", "AGPR"), ("TotalSGPRs", "SGPR"), ("VGPRs Spill", "VGPR spill"),
           ("SGPRs Spill", "SGPR spill"), ("ScratchSize [bytes/lane]", "scratch B/lane"),
           ("LDS Size [bytes/block]", "LDS B/block"), ("Occupancy [waves/SIMD]", "waves/SIMD")]


def _demangle(names):
    r = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True, text=True)
    out = r.stdout.splitlines() if r.returncode == 0 else []
    return out if len(out) == len(names) else list(names)


def resource_usage(out_path):
    """Write the compiler's per-kernel resource report of every device source."""
    os.makedirs(BUILD, exist_ok=True)
    rows = []
    for src in (s for s in SOURCES if s.endswith(".hip")):
        msgs = _compile(src, False, ["-Rpass-analysis=kernel-resource-usage"],
                        os.path.join(BUILD, src + ".ru.o"))
        cur = None
        for ln in msgs:
            m = re.search(r"remark:\s+(.*?): (.*?) \[-Rpass-analysis", ln)
            if not m:
                continue
            key, val = m.group(1).strip(), m.group(2).strip()
            if key == "Function Name":
                cur = {"src": src, "name": val}
                rows.append(cur)
            elif cur is not None:
                cur[key] = val
    names = _demangle([r["name"] for r in rows])
    lines = ["| source | kernel | " + " | ".join(h for _, h in _FIELDS) + " |",
             "|---|---|" + "---|" * len(_FIELDS)]
    for r, n in zip(rows, names):
        n = re.sub(r"^jfa::\(anonymous namespace\)::", "", n)
        n = re.sub(r"\(jfa::[A-Za-z]+Params\)$", "", n)
        lines.append(f"| {r['src']} | `{n}` | " + " | ".join(r.get(k, "") for k, _ in _FIELDS) + " |")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return out_path


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
    if "--resource-usage" in sys.argv:
        print(resource_usage(sys.argv[sys.argv.index("--resource-usage") + 1]))
    else:
        print(build(verbose="-v" in sys.argv))
