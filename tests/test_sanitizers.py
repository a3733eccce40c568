"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two executables are built in a temporary directory and must run clean:
- the fp64 oracle (oracle/oracle.c) driven through every entry point on small
  dense and block-sparse problems (tests/sanitize/oracle_main.c), with gcc;
- the C ABI's host code (fa2_api.hip) driven through every argument check
  that returns before a HIP call (tests/sanitize/validators_main.cpp).  Only
  the host side is instrumented (each -fsanitize= follows -Xarch_host); the
  kernel launchers are replaced by stand-ins that abort if reached.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "exact_io_aware_26_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
HIPCC = "/opt/rocm/bin/hipcc"
CLANGXX = "/opt/rocm/llvm/bin/clang++"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc missing")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-o", exe, os.path.join(SAN, "oracle_main.c"),
          os.path.join(ROOT, "oracle", "oracle.c"), "-lm"])
    r = _run([exe], env=dict(ENV, ASAN_OPTIONS="detect_leaks=1"))
    assert "oracle ok" in r.stdout


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)), reason="ROCm toolchain missing")
def test_abi_validators_under_asan_and_ubsan(tmp_path):
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all"]
    common = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature",
              "-Xclang", "-packed-fp32-ops", "-I", INCLUDE, "-I", CSRC]
    api, stubs, main = (str(tmp_path / n) for n in ("api.o", "stubs.o", "main.o"))
    _run([HIPCC, *common, *host_san, "-c", os.path.join(CSRC, "fa2_api.hip"), "-o", api])
    _run([HIPCC, *common, "-x", "hip", *host_san, "-c", os.path.join(SAN, "launch_stubs.cpp"), "-o", stubs])
    _run([CLANGXX, "-g", "-std=c++17", "-I", INCLUDE, "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-c", os.path.join(SAN, "validators_main.cpp"), "-o", main])
    exe = str(tmp_path / "validators")
    _run([CLANGXX, "-fsanitize=address,undefined", api, stubs, main, "-L/opt/rocm/lib",
          "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64", "-o", exe])
    r = _run([exe], env=ENV)
    assert "validators ok" in r.stdout
