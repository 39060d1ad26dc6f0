"""CPU builds under AddressSanitizer and UndefinedBehaviorSanitizer.

* The float64 oracle (oracle/gdn_oracle.c) with gcc, driven by
  tests/native/oracle_sanitize.c: packed batches with empty and one-token
  sequences, grouped heads, several thread counts, its argument checks.
* The C ABI's host code (gated_deltanet_02_amd/csrc/gdn_api.cpp: argument
  validation, workspace layouts, options, the cu_seqlens validator, the
  graph cache's bookkeeping) with hipcc's host compiler, linked with
  host-only stand-ins for the launchers and the HIP runtime
  (tests/native/api_stubs.cpp) and driven by tests/native/api_sanitize.cpp.
  No GPU code is built; the sanitizers apply to host code only.
A sanitizer report makes the test program exit non-zero.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
CSRC = os.path.join(ROOT, "gated_deltanet_02_amd", "csrc")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:abort_on_error=0",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{cmd[0]} failed ({r.returncode}):\n{r.stdout}\n{r.stderr[-4000:]}"
    return r


def test_oracle_under_sanitizers(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("gcc not found")
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-O1", "-g", "-std=c99", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", os.path.join(NATIVE, "oracle_sanitize.c"),
          os.path.join(ROOT, "oracle", "gdn_oracle.c"), "-o", exe, "-lm", "-pthread"])
    r = _run([exe], env=ENV, timeout=300)
    assert "0 failure(s)" in r.stdout


def test_host_api_under_sanitizers(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not found")
    exe = str(tmp_path / "api_san")
    _run([hipcc, "-O1", "-g", "-std=c++17",
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
          f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
          os.path.join(CSRC, "gdn_api.cpp"), os.path.join(NATIVE, "api_stubs.cpp"),
          os.path.join(NATIVE, "api_sanitize.cpp"), "-o", exe], timeout=600)
    r = _run([exe], env=ENV, timeout=300)
    assert "0 failure(s)" in r.stdout
