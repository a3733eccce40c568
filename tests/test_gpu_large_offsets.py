"""Tensors past 2^31 elements: 64-bit offsets in every kernel.

B=64, Hq=128 (GQA onto 64 K/V heads), N=2048, d=128 gives 2^31 elements (4 GiB in
bf16) per query-side tensor, so the element offsets of the last heads exceed
2^31 and their byte offsets 2^32.  The work is only 8192 short heads, so the
GPU part takes milliseconds.  Inputs are seeded N(0,1) bf16 drawn on the
device; the heads checked are copied back and compared in full with the fp64
oracle (forward and backward), as in the other GPU tests.
"""
import math

import numpy as np
import pytest

from oracle import oracle as orc
from tests import parity
from tests.parity import log

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from exact_io_aware_26_amd import fa2
    fa2.load()


def _f64(t):
    return t.detach().float().double().cpu().numpy()


def test_offsets_past_2_31_elements():
    from exact_io_aware_26_amd import fa2
    B, Hq, Hkv, N, d, causal = 64, 128, 64, 2048, 128, True
    assert B * Hq * N * d == 2 ** 31
    dev = torch.device("cuda:0")
    log(f"[large] B={B} Hq={Hq} Hkv={Hkv} N={N} d={d}: {B * Hq * N * d} elements per query-side tensor")
    g = torch.Generator(device=dev).manual_seed(8)
    q = torch.randn(B, Hq, N, d, device=dev, dtype=torch.bfloat16, generator=g)
    k = torch.randn(B, Hkv, N, d, device=dev, dtype=torch.bfloat16, generator=g)
    v = torch.randn(B, Hkv, N, d, device=dev, dtype=torch.bfloat16, generator=g)
    do = torch.randn(B, Hq, N, d, device=dev, dtype=torch.bfloat16, generator=g)
    o, L = fa2.forward(q, k, v, causal=causal)
    dq, dk, dv = fa2.backward(q, k, v, o, L, do, causal=causal)
    torch.cuda.synchronize()
    sc = 1.0 / math.sqrt(d)
    G = Hq // Hkv
    # The last K/V head (its two query heads end at the last element), one in the middle, the first.
    for b, hk in ((B - 1, Hkv - 1), (B // 2, Hkv // 2 + 3), (0, 0)):
        log(f"[large] checking batch {b}, K/V head {hk} (query heads {hk * G}..{hk * G + G - 1})")
        hs = slice(hk * G, hk * G + G)
        q64, do64 = _f64(q[b:b + 1, hs]), _f64(do[b:b + 1, hs])
        k64, v64 = _f64(k[b:b + 1, hk:hk + 1]), _f64(v[b:b + 1, hk:hk + 1])
        ro, rL = orc.forward(q64, k64, v64, causal, sc)
        parity.check_bf16("O", _f64(o[b:b + 1, hs]), ro)
        parity.check_lse("L", _f64(L[b:b + 1, hs]), rL)
        rdq, rdk, rdv, _ = orc.backward(q64, k64, v64, do64, causal, sc)
        wdq, wdk, wdv = orc.backward_bf16(q64, k64, v64, do64, causal, sc)
        parity.check_bf16("dQ", _f64(dq[b:b + 1, hs]), rdq, working=wdq)
        parity.check_bf16("dK", _f64(dk[b:b + 1, hk:hk + 1]), rdk, working=wdk)
        parity.check_bf16("dV", _f64(dv[b:b + 1, hk:hk + 1]), rdv, working=wdv)
    for name, t in (("O", o), ("dQ", dq), ("dK", dk), ("dV", dv)):
        assert bool(torch.isfinite(t).all()), f"{name} has unwritten or non-finite elements"
    assert bool(torch.isfinite(L).all())
