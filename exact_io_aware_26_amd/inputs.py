"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle side.

This module holds no attention arithmetic: it draws numbers and rounds them
to bfloat16 (or, for the f16 entry points, to IEEE binary16).  Both the HIP path and the CPU oracle receive exactly the arrays
it returns (the oracle as their exact float64 values).

Recipe: NumPy PCG64 ``default_rng(seed)``, ``standard_normal(shape,
dtype=float32)`` drawn in the order the caller lists the tensors (Q, K, V,
then dO), each rounded to bfloat16 with round-to-nearest-even on the upper 16
bits (f16: NumPy's float32 -> float16 conversion, also round-to-nearest-even).
N(0, 1) values never round to NaN or Inf.
"""
from __future__ import annotations

import numpy as np


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    nan = np.isnan(x)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns (uint16) to float32."""
    b = np.ascontiguousarray(np.asarray(b, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(b).astype(np.float64)


def seeded_bf16(seed: int, shapes) -> list[np.ndarray]:
    """Draw one N(0,1) float32 tensor per shape from one PCG64 stream, rounded to bf16 bits."""
    rng = np.random.default_rng(seed)
    out = []
    for shape in shapes:
        x = rng.standard_normal(tuple(shape), dtype=np.float32)
        out.append(f32_to_bf16_bits(x))
    return out


def f16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact widening of IEEE binary16 bit patterns (uint16) to float64."""
    return np.ascontiguousarray(np.asarray(b, dtype=np.uint16)).view(np.float16).astype(np.float64)


def seeded_f16(seed: int, shapes) -> list[np.ndarray]:
    """The same draws as ``seeded_bf16``, rounded to binary16 bits instead."""
    rng = np.random.default_rng(seed)
    return [rng.standard_normal(tuple(shape), dtype=np.float32).astype(np.float16).view(np.uint16)
            for shape in shapes]


def attention_inputs(seed: int, B: int, Hq: int, Hkv: int, N: int, d: int,
                     with_grad: bool = False, fmt: str = "bf16") -> list[np.ndarray]:
    """Bit arrays (uint16) Q [B,Hq,N,d], K, V [B,Hkv,N,d] (and dO [B,Hq,N,d]),
    in bf16 (``fmt="bf16"``) or binary16 (``fmt="f16"``)."""
    shapes = [(B, Hq, N, d), (B, Hkv, N, d), (B, Hkv, N, d)]
    if with_grad:
        shapes.append((B, Hq, N, d))
    if fmt == "f16":
        return seeded_f16(seed, shapes)
    if fmt != "bf16":
        raise ValueError(f"unknown element format {fmt!r}")
    return seeded_bf16(seed, shapes)


SPARSE_BLOCK = 128   # query rows and keys per block-sparse mask block


def block_mask(kind: str, N: int, seed: int = 0, density: float = 0.5, window: int = 4) -> np.ndarray:
    """A block-sparse mask pattern, uint8 [ceil(N/128), ceil(N/128)] (row = query block).

    kind: "ones", "zeros", "diagonal", "column0" (every query block sees key block 0 only),
    "random" (each block kept with probability ``density``, PCG64 ``default_rng(seed)``),
    "local_global" (the ``window`` key blocks ending at the query block's own, plus key
    block 0: a sliding window with one global block), "strided" (key blocks c with
    (r - c) % 4 == 0).
    """
    nb = (N + SPARSE_BLOCK - 1) // SPARSE_BLOCK
    r = np.arange(nb)[:, None]
    c = np.arange(nb)[None, :]
    if kind == "ones":
        m = np.ones((nb, nb), dtype=bool)
    elif kind == "zeros":
        m = np.zeros((nb, nb), dtype=bool)
    elif kind == "diagonal":
        m = r == c
    elif kind == "column0":
        m = np.broadcast_to(c == 0, (nb, nb))
    elif kind == "random":
        m = np.random.default_rng(seed).random((nb, nb)) < density
    elif kind == "local_global":
        m = ((c <= r) & (c > r - window)) | (c == 0)
    elif kind == "strided":
        m = (r - c) % 4 == 0
    else:
        raise ValueError(f"unknown block mask kind {kind!r}")
    return np.ascontiguousarray(m, dtype=np.uint8)
