"""Build libfa2.so (the gfx950 HIP kernels and the C ABI) in-tree with hipcc.

Every translation unit is compiled for gfx950 only, with packed-FP32 VALU
instructions disabled and hardware fp32 atomics enabled, then linked into
``exact_io_aware_26_amd/libfa2.so``.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libfa2.so")
BUILD_DIR = os.path.join(PKG, "_build")
SOURCES = ["fa2_api.hip", "fa2_fwd.hip", "fa2_bwd.hip"]
# Translation units: (source, extra defines, object name).  The kernel sources
# are compiled twice: for bf16 elements (namespace fa2) and for f16 (fa2_f16).
UNITS = [("fa2_api.hip", [], "fa2_api"),
         ("fa2_fwd.hip", [], "fa2_fwd"), ("fa2_bwd.hip", [], "fa2_bwd"),
         ("fa2_fwd.hip", ["-DFA2_F16=1"], "fa2_fwd_f16"), ("fa2_bwd.hip", ["-DFA2_F16=1"], "fa2_bwd_f16")]
# Per-source code generation options.  The kernels feed matrix-core results
# straight into vector arithmetic; with this option the compiler keeps those
# results in ordinary VGPRs instead of accumulation registers that would have
# to be copied out first (the d = 64 / 128 forward kernels compile to the same
# code either way).
SOURCE_FLAGS = {"fa2_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-mllvm", "-pragma-unroll-threshold=1000000"],
                "fa2_fwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics", "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfa2.so)")


def _compile(unit, extra: list[str]) -> str:
    src, defines, name = unit
    obj = os.path.join(BUILD_DIR, name + ".o")
    cmd = [hipcc(), *FLAGS, *SOURCE_FLAGS.get(src, []), *defines, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that warning is expected.
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(extra: list[str] | None = None) -> str:
    """Compile all sources in parallel and link libfa2.so; returns its path."""
    extra = list(extra or [])
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(UNITS)) as ex:
        objs = list(ex.map(lambda u: _compile(u, extra), UNITS))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(sys.argv[1:]))
