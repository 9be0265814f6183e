"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The CPU oracle (oracle/oracle.c), built with gcc and both sanitizers, runs
  every entry point on small ragged inputs held in buffers of exactly their
  documented sizes (tests/sanitize/oracle_driver.c).
* The C ABI's host code (the four HIP sources; only the host half is
  instrumented, the gfx950 code is built as usual) is driven through its
  argument validation with invalid calls that must all be refused before any
  device work (tests/sanitize/abi_driver.c); no GPU is needed.

Any out-of-bounds access, use after free, signed overflow or other undefined
behaviour aborts the driver and fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "block_sparse_int8_amd", "csrc")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
           OMP_NUM_THREADS="2")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not installed")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp", "-ffp-contract=off",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(SAN, "oracle_driver.c"), "-lm", "-o", exe])
    r = _run([exe], env=ENV)
    assert "all cases ran" in r.stdout


HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm compilers not installed")
def test_abi_validation_under_asan_ubsan(tmp_path):
    lib = str(tmp_path / "libsparse_attn.so")
    # sanitizers on the host half only: each -fsanitize= follows -Xarch_host
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument",
          *host_san, "-I", os.path.join(ROOT, "include"),
          *[os.path.join(CSRC, s) for s in ("abi.hip", "quantize.hip", "route.hip", "fwd.hip")], "-o", lib])
    exe = str(tmp_path / "abi_driver")
    _run([CLANG, "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"), os.path.join(SAN, "abi_driver.c"),
          lib, "-Wl,-rpath," + str(tmp_path), "-o", exe])
    r = _run([exe], env=ENV)
    assert "every invalid call refused" in r.stdout
