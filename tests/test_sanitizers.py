"""The oracle and the host side of the C ABI built with AddressSanitizer and
UndefinedBehaviorSanitizer and driven on the CPU (no GPU needed).

* ``oracle/tlsl_oracle.c`` with ``tests/native/oracle_driver.c``: every oracle
  entry point on the DSA page's worked example and a seeded random case.
* ``csrc/abi.cpp`` + ``csrc/plan.cpp`` (argument validation, workspace sizing
  and layouts) with the launcher stand-ins of ``tests/native/abi_stubs.cpp``
  and ``tests/native/abi_driver.cpp``: every entry point through its error,
  size-query and accepted paths.

A sanitizer report aborts the driver (``-fno-sanitize-recover=all``), which
fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
CSRC = os.path.join(ROOT, "token_level_sparse_lightning_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c11", "-fopenmp", "-ffp-contract=off", *SAN,
          os.path.join(ROOT, "oracle", "tlsl_oracle.c"), os.path.join(NATIVE, "oracle_driver.c"),
          "-o", exe, "-lm"], ROOT)
    r = subprocess.run([exe], capture_output=True, text=True, env=dict(ENV, OMP_NUM_THREADS="4"))
    assert r.returncode == 0 and "oracle driver ok" in r.stdout, r.stdout + r.stderr


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="g++ or the ROCm headers not available")
def test_host_abi_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "abi_driver")
    _run(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", f"-I{os.path.join(ROOT, 'include')}",
          *SAN, os.path.join(CSRC, "abi.cpp"), os.path.join(CSRC, "plan.cpp"),
          os.path.join(NATIVE, "abi_stubs.cpp"), os.path.join(NATIVE, "abi_driver.cpp"), "-o", exe], ROOT)
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV)
    assert r.returncode == 0 and "abi driver ok" in r.stdout, r.stdout + r.stderr
