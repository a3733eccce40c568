"""NumPy binding of the fp64 CPU attention oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this module; the product path never does.

The oracle evaluates the plain definition of exact attention
(O = softmax(scale * Q K^T [+ causal mask]) V, per-row logsumexp L, and the
gradients dQ, dK, dV of sum(dO * O)) in double precision, following the
FlashAttention-2 summary page (zhaifeiyue.github.io), section 3 "Target
operation" and section 4's symbol table and checks.  Every function takes
float64 arrays in [B, H, N, d] layout (any values; bf16 inputs are passed as
their exact float64 values).  ``block_mask`` (optional, every function):
a [ceil(N/128), ceil(N/128)] array, nonzero where a 128-row block of queries
may attend to a 128-key block (block-sparse attention, shared by all batches
and heads); see oracle.c for the convention on rows it masks entirely.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True, src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile ``oracle.c`` with gcc (-O2, OpenMP, no fast-math) into a shared library."""
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(src):
        return out
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall",
           "-o", out + ".tmp", src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _open(path: str):
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int)
    i = ctypes.c_int
    bm = ctypes.c_void_p          # block mask bytes, or None
    lib.oracle_fwd.argtypes = [dp, dp, dp, dp, dp, i, i, i, i, i, i, bm, ctypes.c_double]
    lib.oracle_fwd_rows.argtypes = [dp, dp, dp, i, i, i, i, i, i, bm, ctypes.c_double,
                                    i, ip, ip, ip, dp, dp]
    lib.oracle_bwd.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, i, i, i, i, i, i, bm,
                               ctypes.c_double]
    lib.oracle_bwd_head.argtypes = [dp, dp, dp, dp, i, i, i, i, i, i, bm, ctypes.c_double,
                                    i, i, dp, dp, dp, dp, dp]
    lib.oracle_bwd_given.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, dp, i, i, i, i, i, i, bm,
                                     ctypes.c_double]
    lib.oracle_bwd_given_bf16.argtypes = lib.oracle_bwd_given.argtypes
    lib.oracle_fwd_bf16.argtypes = [dp, dp, dp, dp, dp, i, i, i, i, i, i, bm, ctypes.c_double]
    lib.oracle_bwd_bf16.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, i, i, i, i, i, i, bm,
                                    ctypes.c_double]
    lib.oracle_bwd_bf16_head.argtypes = [dp, dp, dp, dp, i, i, i, i, i, i, bm, ctypes.c_double,
                                         i, i, dp, dp, dp]
    for f in (lib.oracle_fwd, lib.oracle_fwd_rows, lib.oracle_bwd, lib.oracle_bwd_head, lib.oracle_bwd_given,
              lib.oracle_bwd_given_bf16,
              lib.oracle_fwd_bf16, lib.oracle_bwd_bf16, lib.oracle_bwd_bf16_head):
        f.restype = ctypes.c_int
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    return lib


def load(path: str | None = None):
    """Load and type the oracle library.

    With no ``path``: the in-tree ``liboracle.so``, built first if absent or
    older than ``oracle.c``, cached after the first call.  With a ``path``: that
    library (used by tests that build deliberately broken copies).
    """
    global _lib
    if path is not None:
        return _open(path)
    if _lib is None:
        _lib = _open(build(force=False))
    return _lib


def _f64(x) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    return a


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _dims(q: np.ndarray, k: np.ndarray):
    B, Hq, N, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if (Bk, Nk, dk) != (B, N, d):
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape}")
    return B, Hq, Hkv, N, d


SPARSE_BLOCK = 128   # rows and keys per block of a block-sparse mask


def _mask(block_mask, N: int):
    """Block mask as contiguous uint8 [ceil(N/128), ceil(N/128)] (None: dense)."""
    if block_mask is None:
        return None
    nb = (N + SPARSE_BLOCK - 1) // SPARSE_BLOCK
    m = np.ascontiguousarray(np.asarray(block_mask) != 0, dtype=np.uint8)
    if m.shape != (nb, nb):
        raise ValueError(f"block mask shape {m.shape}, expected {(nb, nb)}")
    return m


def _mptr(m):
    return None if m is None else m.ctypes.data


def default_scale(d: int) -> float:
    return 1.0 / np.sqrt(d)


def num_threads(lib=None) -> int:
    return (lib or load()).oracle_num_threads()


def forward(q, k, v, causal: bool = False, scale: float | None = None, lib=None, block_mask=None):
    """Full forward: returns (O [B,Hq,N,d], L [B,Hq,N]) in float64."""
    lib = lib or load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Hkv, N, d = _dims(q, k)
    bm = _mask(block_mask, N)
    if scale is None:
        scale = default_scale(d)
    o = np.empty_like(q)
    L = np.empty((B, Hq, N), dtype=np.float64)
    rc = lib.oracle_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(L),
                        B, Hq, Hkv, N, d, int(causal), _mptr(bm), float(scale))
    if rc != 0:
        raise ValueError("oracle_fwd: bad sizes")
    return o, L


def forward_rows(q, k, v, rows, causal: bool = False, scale: float | None = None, lib=None, block_mask=None):
    """Forward for selected rows.  ``rows`` is an int array [n, 3] of (b, hq, i).

    Returns (O_rows [n, d], L_rows [n]) in float64.
    """
    lib = lib or load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Hkv, N, d = _dims(q, k)
    bm = _mask(block_mask, N)
    if scale is None:
        scale = default_scale(d)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 3))
    rb = np.ascontiguousarray(rows[:, 0])
    rh = np.ascontiguousarray(rows[:, 1])
    ri = np.ascontiguousarray(rows[:, 2])
    n = rows.shape[0]
    o = np.empty((n, d), dtype=np.float64)
    L = np.empty((n,), dtype=np.float64)
    ip = ctypes.POINTER(ctypes.c_int)
    rc = lib.oracle_fwd_rows(_ptr(q), _ptr(k), _ptr(v), B, Hq, Hkv, N, d, int(causal), _mptr(bm),
                             float(scale), n, rb.ctypes.data_as(ip), rh.ctypes.data_as(ip),
                             ri.ctypes.data_as(ip), _ptr(o), _ptr(L))
    if rc != 0:
        raise ValueError("oracle_fwd_rows: bad sizes or row index")
    return o, L


def backward(q, k, v, do, causal: bool = False, scale: float | None = None, lib=None, block_mask=None):
    """Full backward: returns (dQ, dK, dV, D) in float64 (D is [B,Hq,N])."""
    lib = lib or load()
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, Hq, Hkv, N, d = _dims(q, k)
    bm = _mask(block_mask, N)
    if scale is None:
        scale = default_scale(d)
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    D = np.empty((B, Hq, N), dtype=np.float64)
    rc = lib.oracle_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv),
                        _ptr(D), B, Hq, Hkv, N, d, int(causal), _mptr(bm), float(scale))
    if rc != 0:
        raise ValueError("oracle_bwd: bad sizes")
    return dq, dk, dv, D


def backward_head(q, k, v, do, b: int, hk: int, causal: bool = False,
                  scale: float | None = None, lib=None, block_mask=None):
    """Backward of key/value head (b, hk) only.

    Returns (dQ [G,N,d] for query heads hk*G.., dK [N,d], dV [N,d], L [G,N], D [G,N]).
    """
    lib = lib or load()
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, Hq, Hkv, N, d = _dims(q, k)
    bm = _mask(block_mask, N)
    G = Hq // Hkv
    if scale is None:
        scale = default_scale(d)
    dq = np.empty((G, N, d), dtype=np.float64)
    dk = np.empty((N, d), dtype=np.float64)
    dv = np.empty((N, d), dtype=np.float64)
    L = np.empty((G, N), dtype=np.float64)
    D = np.empty((G, N), dtype=np.float64)
    rc = lib.oracle_bwd_head(_ptr(q), _ptr(k), _ptr(v), _ptr(do), B, Hq, Hkv, N, d,
                             int(causal), _mptr(bm), float(scale), int(b), int(hk), _ptr(dq),
                             _ptr(dk), _ptr(dv), _ptr(L), _ptr(D))
    if rc != 0:
        raise ValueError("oracle_bwd_head: bad sizes or head index")
    return dq, dk, dv, L, D


def backward_given(q, k, v, o, L, do, causal: bool = False, scale: float | None = None, lib=None,
                   block_mask=None, working_precision: bool = False):
    """The backward from given forward outputs o [B,Hq,N,d] and L [B,Hq,N]:
    P = exp(S - L), D = rowsum(do * o) from the given o.  Returns (dQ, dK, dV).
    ``working_precision``: P and dS rounded to bf16 before their products (the
    method's operand precision), results unrounded."""
    lib = lib or load()
    q, k, v, o, L, do = _f64(q), _f64(k), _f64(v), _f64(o), _f64(L), _f64(do)
    B, Hq, Hkv, N, d = _dims(q, k)
    if o.shape != q.shape or do.shape != q.shape or L.shape != (B, Hq, N):
        raise ValueError("o and do must be shaped like q, L like [B, Hq, N]")
    bm = _mask(block_mask, N)
    if scale is None:
        scale = default_scale(d)
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    fn = lib.oracle_bwd_given_bf16 if working_precision else lib.oracle_bwd_given
    rc = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(L), _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv),
            B, Hq, Hkv, N, d, int(causal), _mptr(bm), float(scale))
    if rc != 0:
        raise ValueError("oracle_bwd_given: bad sizes")
    return dq, dk, dv


def forward_bf16(q, k, v, causal: bool = False, scale: float | None = None, lib=None, block_mask=None):
    """The forward at the method's working precision (bf16 P in P V): (O unrounded, L)."""
    lib = lib or load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Hkv, N, d = _dims(q, k)
    bm = _mask(block_mask, N)
    if scale is None:
        scale = default_scale(d)
    o = np.empty_like(q)
    L = np.empty((B, Hq, N), dtype=np.float64)
    rc = lib.oracle_fwd_bf16(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(L),
                             B, Hq, Hkv, N, d, int(causal), _mptr(bm), float(scale))
    if rc != 0:
        raise ValueError("oracle_fwd_bf16: bad sizes")
    return o, L


def backward_bf16(q, k, v, do, causal: bool = False, scale: float | None = None, lib=None, block_mask=None,
                  return_d: bool = False):
    """The backward at the method's working precision: (dQ, dK, dV) unrounded (and D)."""
    lib = lib or load()
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, Hq, Hkv, N, d = _dims(q, k)
    bm = _mask(block_mask, N)
    if scale is None:
        scale = default_scale(d)
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    D = np.empty((B, Hq, N), dtype=np.float64)
    rc = lib.oracle_bwd_bf16(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv),
                             _ptr(D), B, Hq, Hkv, N, d, int(causal), _mptr(bm), float(scale))
    if rc != 0:
        raise ValueError("oracle_bwd_bf16: bad sizes")
    return (dq, dk, dv, D) if return_d else (dq, dk, dv)


def backward_bf16_head(q, k, v, do, b: int, hk: int, causal: bool = False,
                       scale: float | None = None, lib=None, block_mask=None):
    """Working-precision backward of key/value head (b, hk): (dQ [G,N,d], dK [N,d], dV [N,d])."""
    lib = lib or load()
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, Hq, Hkv, N, d = _dims(q, k)
    bm = _mask(block_mask, N)
    G = Hq // Hkv
    if scale is None:
        scale = default_scale(d)
    dq = np.empty((G, N, d), dtype=np.float64)
    dk = np.empty((N, d), dtype=np.float64)
    dv = np.empty((N, d), dtype=np.float64)
    rc = lib.oracle_bwd_bf16_head(_ptr(q), _ptr(k), _ptr(v), _ptr(do), B, Hq, Hkv, N, d,
                                  int(causal), _mptr(bm), float(scale), int(b), int(hk), _ptr(dq),
                                  _ptr(dk), _ptr(dv))
    if rc != 0:
        raise ValueError("oracle_bwd_bf16_head: bad sizes or head index")
    return dq, dk, dv
