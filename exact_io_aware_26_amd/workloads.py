"""Named attention workloads and their FLOP accounting.

The FLOP convention is the one the FlashAttention-2 summary page
(zhaifeiyue.github.io) gives in section 3 ("FLOPs"): a forward pass costs
4 * N^2 * d per head (two matmuls), half that with a causal mask, and the
backward pass costs 2.5 times the forward (five matmuls instead of two).
Batch is a plain multiplier.  Query heads are counted (GQA shares K/V heads
but each query head still does the full work).
"""
from __future__ import annotations

import dataclasses
import math


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    causal: bool
    seed: int
    backward: bool = False

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def fwd_flops(self) -> float:
        f = 4.0 * self.B * self.Hq * self.N * self.N * self.d
        return f / 2.0 if self.causal else f

    def bwd_flops(self) -> float:
        return 2.5 * self.fwd_flops()

    def as_dict(self) -> dict:
        return dataclasses.asdict(self)


# The five workloads the method is benchmarked on, by what they are.
TINY = Workload("tiny_fwd_b1_h1_n128_d64", 1, 1, 1, 128, 64, False, seed=1)
SHORT_NONCAUSAL = Workload("fwd_short_b8_h16_n2048_d64", 8, 16, 16, 2048, 64, False, seed=2)
SHORT_CAUSAL = Workload("fwd_short_causal_b8_h16_n2048_d64", 8, 16, 16, 2048, 64, True, seed=2)
LONG = Workload("fwd_long_causal_b2_h16_n16384_d128", 2, 16, 16, 16384, 128, True, seed=3)
GQA_D128 = Workload("fwd_gqa_causal_b4_hq32_hkv8_n4096_d128", 4, 32, 8, 4096, 128, True, seed=4)
GQA_D256 = Workload("fwd_gqa_causal_b4_hq32_hkv8_n4096_d256", 4, 32, 8, 4096, 256, True, seed=4)
BWD = Workload("fwd_bwd_causal_b4_h16_n8192_d128", 4, 16, 16, 8192, 128, True, seed=5,
               backward=True)

ALL = [TINY, SHORT_NONCAUSAL, SHORT_CAUSAL, LONG, GQA_D128, GQA_D256, BWD]
BY_NAME = {w.name: w for w in ALL}


def block_sparse_fwd_flops(mask, B: int, Hq: int, N: int, d: int, causal: bool) -> float:
    """Forward FLOPs of block-sparse attention in the same convention: 4 * d per
    (query, key) pair of every kept 128 x 128 block, a block on the causal
    diagonal counted as half its pairs (as the dense causal count halves N^2).
    The backward is 2.5 times this."""
    import numpy as np
    bs = 128
    m = np.asarray(mask) != 0
    nb = m.shape[0]
    size = np.minimum(bs, N - bs * np.arange(nb)).astype(np.float64)   # rows (= keys) per block
    pairs = np.outer(size, size)
    if causal:
        r, c = np.indices((nb, nb))
        pairs = np.where(c < r, pairs, np.where(c == r, pairs / 2.0, 0.0))
    return 4.0 * B * Hq * d * float(np.sum(pairs[m]))
