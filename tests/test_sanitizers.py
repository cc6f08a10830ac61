"""Host-only AddressSanitizer and UndefinedBehaviorSanitizer runs (no GPU needed):

- the CPU oracle (plain C), exercised by tests/sanitize/oracle_exercise.c over every shape class and
  its argument errors;
- the C ABI's host side (validation, planning, workspace sizes: csrc/capi.hip compiled with the
  sanitizers on its host pass only; the device code and the other objects are the library's
  own), exercised by tests/sanitize/capi_exercise.cpp: valid shapes of every path, a pseudo-random
  sweep of 200,000 parameter sets with sizes up to 2^40, and every entry point's argument and
  workspace errors, which return before any HIP call.

A sanitizer report makes the program exit non-zero (no recovery) and fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "sparse_transformer_attention_amd", "csrc")
OBJDIR = os.path.join(ROOT, "sparse_transformer_attention_amd", "_build")
ROCM = "/opt/rocm"
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="2")


def _run(exe):
    res = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=SAN_ENV)
    report = res.stdout[-3000:] + res.stderr[-3000:]
    assert res.returncode == 0, report
    assert "ERROR: AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr, report
    assert "all checks passed" in res.stdout, report


def test_oracle_under_asan_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    exe = str(tmp_path / "oracle_exercise")
    subprocess.check_call(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fopenmp",
                           os.path.join(SAN, "oracle_exercise.c"),
                           os.path.join(ROOT, "oracle", "condensate_oracle.c"), "-lm", "-o", exe])
    _run(exe)


def test_capi_host_side_under_asan_ubsan(tmp_path):
    hipcc, clangxx = os.path.join(ROCM, "bin", "hipcc"), os.path.join(ROCM, "llvm", "bin", "clang++")
    if not (os.path.exists(hipcc) and os.path.exists(clangxx)):
        pytest.skip("ROCm compilers not found")
    others = sorted(os.path.join(OBJDIR, f) for f in os.listdir(OBJDIR)
                    if f.endswith(".hip.o") and f != "capi.hip.o") if os.path.isdir(OBJDIR) else []
    if not others:
        pytest.skip("library objects not built (run __graft_entry__.build() first)")
    capi_o, ex_o, exe = (str(tmp_path / n) for n in ("capi.o", "exercise.o", "capi_exercise"))
    # Sanitizers on the host pass only: each -fsanitize flag behind its own -Xarch_host.
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    subprocess.run([hipcc, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    "-I", os.path.join(ROOT, "include"), "-I", CSRC, *host_san,
                    "-c", os.path.join(CSRC, "capi.hip"), "-o", capi_o],
                   check=True, capture_output=True, text=True)
    subprocess.check_call([clangxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"),
                           "-c", os.path.join(SAN, "capi_exercise.cpp"), "-o", ex_o])
    subprocess.check_call([clangxx, "-fsanitize=address,undefined", "-o", exe, ex_o, capi_o, *others,
                           "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                           "-Wl,-rpath," + os.path.join(ROCM, "lib")])
    _run(exe)
