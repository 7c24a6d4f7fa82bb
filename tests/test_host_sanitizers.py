"""The host runtime under AddressSanitizer and UndefinedBehaviorSanitizer.

jfa_api.cpp and jfa_sched.cpp size every workspace region, tile list and capacity
that the kernels later write through; a host-side overflow there would go unseen on
the GPU.  This test rebuilds those two files with g++ -fsanitize=address,undefined
(host code only: the device objects of the normal build are linked in unchanged and
no kernel runs), then runs the ABI and schedule-specification tests against that
library in a child process with the sanitizer runtime preloaded.  Any sanitizer report
fails the run (UB is made fatal, ASan aborts on error)."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "variable_length_flash_jagged_amd")
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
HOST_SOURCES = ["jfa_api.cpp", "jfa_sched.cpp"]


def _device_objects():
    from variable_length_flash_jagged_amd import build as bld
    objs = [os.path.join(BUILD, s + ".o") for s in bld.SOURCES if s.endswith(".hip")]
    if not all(os.path.exists(o) for o in objs):
        bld.build()
    return objs


def _runtime(name):
    r = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_abi_and_schedule_tests_clean_under_asan_and_ubsan(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("no libasan runtime for g++")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    flags = ["-std=c++17", "-O1", "-g", "-fPIC", "-fno-omit-frame-pointer",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             # std::vector accesses past size() (within capacity) and operator[] range checks
             "-D_GLIBCXX_SANITIZE_VECTOR", "-D_GLIBCXX_ASSERTIONS",
             "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"),
             "-I", CSRC]
    objs = []
    for src in HOST_SOURCES:
        obj = str(tmp_path / (src + ".o"))
        r = subprocess.run(["g++"] + flags + ["-c", os.path.join(CSRC, src), "-o", obj], capture_output=True,
                           text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        objs.append(obj)
    lib = str(tmp_path / "libjfa_sanitized.so")
    r = subprocess.run(["g++", "-shared", "-fsanitize=address,undefined", "-o", lib] + objs + _device_objects()
                       + ["-L", os.path.join(rocm, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(rocm, "lib")],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    nm = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in nm and "__ubsan_handle" in nm, "library is not instrumented"

    env = dict(os.environ)
    env.update(JFA_LIBRARY=lib, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:detect_odr_violation=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    check = ("from variable_length_flash_jagged_amd import binding as B; "
             f"assert B.LIB_PATH == {lib!r}; B.lib(); print('sanitized library loaded')")
    r = subprocess.run([sys.executable, "-c", check], cwd=ROOT, env=env, capture_output=True, text=True)
    assert r.returncode == 0 and "sanitized library loaded" in r.stdout, r.stdout[-2000:] + r.stderr[-2000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "tests/test_abi.py", "tests/test_schedule_spec.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in out
