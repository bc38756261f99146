"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

A copy of the library is built with the sanitizers on its host code only
(device code as usual) and driven by tests/host_sanitize/exercise_abi.c without a
GPU: argument validation and overlap checks, workspace sizing, the shape-group
plan, launch tables and schedule cache of valid calls (which then fail at their
first HIP call), cache eviction, and the streaming entry points' checks.  Any
sanitizer report ends the test program with a non-zero status.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "muon_optimizer_step_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm compilers not installed")
@pytest.mark.skipif(os.path.exists("/dev/kfd"),
                    reason="the test program's valid calls carry fake device pointers: run only where no GPU is present")
def test_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    lib = tmp_path / "libmuonstep_san.so"
    sources = [os.path.join(CSRC, f) for f in ("api.hip", "elementwise.hip", "ns.hip", "chain.hip")]
    build = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined",
             "-I", os.path.join(ROOT, "include")] + sources + ["-o", str(lib)]
    r = subprocess.run(build, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = tmp_path / "exercise_abi"
    link = [CLANG, "-std=c11", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
            "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"),
            os.path.join(ROOT, "tests", "host_sanitize", "exercise_abi.c"),
            f"-L{tmp_path}", "-lmuonstep_san", f"-Wl,-rpath,{tmp_path}", "-o", str(exe)]
    r = subprocess.run(link, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ)
    # the HIP runtime the library loads is not instrumented and keeps allocations for the process lifetime
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "ALL OK" in r.stdout, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    shutil.rmtree(tmp_path, ignore_errors=True)
