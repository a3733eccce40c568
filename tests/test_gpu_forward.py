"""Forward pass on the GPU against the fp64 oracle, element by element.

Inputs are the seeded bf16 tensors of ``exact_io_aware_26_amd.inputs``; the
oracle receives their exact values.  Outputs are pre-filled with NaN so an
unwritten element fails.  Small shapes are compared in full (several tiles
and ragged tails); the benchmark workloads at full size are compared on
sampled rows, which the oracle computes one at a time.
"""
import math

import numpy as np
import pytest

from exact_io_aware_26_amd import inputs, workloads
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


def run_fwd(qb, kb, vb, causal, scale=None):
    from exact_io_aware_26_amd import fa2
    q, k, v = (parity.to_device_bf16(x) for x in (qb, kb, vb))
    out = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=q.device)
    o, L = fa2.forward(q, k, v, causal=causal, scale=scale, out=out, lse=lse)
    torch.cuda.synchronize()
    return o, L


def full_case(seed, B, Hq, Hkv, N, d, causal, scale=None):
    log(f"[fwd] seed={seed} B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} causal={causal}")
    qb, kb, vb = inputs.attention_inputs(seed, B, Hq, Hkv, N, d)
    o, L = run_fwd(qb, kb, vb, causal, scale)
    q64, k64, v64 = (inputs.bf16_bits_to_f64(x) for x in (qb, kb, vb))
    ro, rL = orc.forward(q64, k64, v64, causal, scale if scale else 1.0 / math.sqrt(d))
    mo = parity.check_bf16("O", parity.bf16_to_f64(o), ro)
    mL = parity.check_lse("L", parity.f32_to_f64(L), rL)
    return mo, mL


SWEEP = []
for N in (1, 2, 17, 63, 64, 65, 127, 128, 130, 257):
    for d in (64, 128, 256):
        for causal in (False, True):
            heads = [(1, 1), (4, 1), (4, 2), (8, 8)][(N + d // 64 + causal) % 4]
            B = 1 + (N % 2)
            SWEEP.append((B, heads[0], heads[1], N, d, causal))


@pytest.mark.parametrize("B,Hq,Hkv,N,d,causal", SWEEP)
def test_fwd_small_sweep(B, Hq, Hkv, N, d, causal):
    full_case(100 + N + d, B, Hq, Hkv, N, d, causal)


@pytest.mark.parametrize("N", [1000, 2048])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_multi_tile(N, d, causal):
    full_case(7, 1, 2, 1, N, d, causal)


def test_fwd_tiny_workload_full():
    w = workloads.TINY
    full_case(w.seed, w.B, w.Hq, w.Hkv, w.N, w.d, w.causal)


def sample_rows(B, Hq, N, n, rng):
    rows = {(0, 0, 0), (B - 1, Hq - 1, N - 1), (0, Hq - 1, N // 2)}
    for t in (63, 64, 127, 128, 129, 255, 256):
        if t < N:
            rows.add((int(rng.integers(B)), int(rng.integers(Hq)), t))
    while len(rows) < n:
        rows.add((int(rng.integers(B)), int(rng.integers(Hq)), int(rng.integers(N))))
    return np.array(sorted(rows), dtype=np.int32)


FWD_WORKLOADS = [workloads.SHORT_NONCAUSAL, workloads.SHORT_CAUSAL, workloads.LONG,
                 workloads.GQA_D128, workloads.GQA_D256, workloads.BWD]


@pytest.mark.parametrize("w", FWD_WORKLOADS, ids=lambda w: w.name)
def test_fwd_workload_sampled_rows(w):
    log(f"[fwd] workload {w.name} (seed {w.seed})")
    qb, kb, vb = inputs.attention_inputs(w.seed, w.B, w.Hq, w.Hkv, w.N, w.d)
    o, L = run_fwd(qb, kb, vb, w.causal)
    Lh = parity.f32_to_f64(L)
    assert np.all(np.isfinite(Lh)), "L has unwritten or non-finite rows"
    # Every O element written and finite (checked on the device to avoid a huge copy).
    assert bool(torch.isfinite(o).all()), "O has unwritten or non-finite elements"
    rows = sample_rows(w.B, w.Hq, w.N, 96, np.random.default_rng(w.seed))
    q64, k64, v64 = (inputs.bf16_bits_to_f64(x) for x in (qb, kb, vb))
    ro, rL = orc.forward_rows(q64, k64, v64, rows, w.causal, w.scale)
    idx = torch.from_numpy(rows.astype(np.int64)).to(o.device)
    og = o[idx[:, 0], idx[:, 1], idx[:, 2]]
    parity.check_bf16("O rows", parity.bf16_to_f64(og), ro)
    parity.check_lse("L rows", Lh[rows[:, 0], rows[:, 1], rows[:, 2]], rL)


# ----------------------------------------------------------------------------- pins on the GPU
def test_fwd_causal_row0_is_v0_bitwise():
    qb, kb, vb = inputs.attention_inputs(21, 2, 4, 2, 300, 128)
    o, L = run_fwd(qb, kb, vb, True)
    v = parity.to_device_bf16(vb)
    G = 2
    for h in range(4):
        assert torch.equal(o[:, h, 0].view(torch.int16), v[:, h // G, 0].view(torch.int16))
    q64, k64 = inputs.bf16_bits_to_f64(qb), inputs.bf16_bits_to_f64(kb)
    L0 = np.einsum("bhd,bhd->bh", q64[:, :, 0], np.repeat(k64, G, axis=1)[:, :, 0]) / math.sqrt(128)
    parity.check_lse("L row 0", parity.f32_to_f64(L[:, :, 0]), L0)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_fwd_zero_queries(d):
    N = 700
    _, kb, vb = inputs.attention_inputs(22, 1, 2, 2, N, d)
    qb = np.zeros((1, 2, N, d), dtype=np.uint16)
    for causal in (False, True):
        o, L = run_fwd(qb, kb, vb, causal)
        cnt = np.arange(1, N + 1) if causal else np.full(N, N)
        parity.check_lse("L (Q=0)", parity.f32_to_f64(L), np.broadcast_to(np.log(cnt), (1, 2, N)))
        v64 = inputs.bf16_bits_to_f64(vb)
        ref = np.cumsum(v64, axis=2) / cnt[None, None, :, None] if causal else \
            np.broadcast_to(v64.mean(axis=2, keepdims=True), v64.shape)
        parity.check_bf16("O (Q=0)", parity.bf16_to_f64(o), ref)


@pytest.mark.parametrize("a,causal", [(0.05, True), (0.05, False), (0.6, True), (3.0, True)])
def test_fwd_geometric_rows_rescale_every_tile(a, causal):
    """S_ij = a*j grows along every row, so the running max moves on every key tile."""
    from tests.oracle_pins import geometric_expected
    N, d = 4000, 64
    j = np.arange(N)
    q = np.zeros((1, 1, N, d), np.float32); q[..., 0] = 2.0 ** -4 * 256; q[..., 1] = 2.0 ** -4
    k = np.zeros((1, 1, N, d), np.float32); k[0, 0, :, 0] = j // 256; k[0, 0, :, 1] = j % 256
    v = np.zeros((1, 1, N, d), np.float32); v[0, 0, :, 0] = (j % 256) / 256.0
    v[0, 0, :, 1] = 1.0
    qb, kb, vb = (inputs.f32_to_bf16_bits(x) for x in (q, k, v))
    assert np.array_equal(inputs.bf16_bits_to_f32(kb), k)   # all values exact in bf16
    o, L = run_fwd(qb, kb, vb, causal, scale=a * 16.0)
    eL, _ = geometric_expected(N, a, causal)
    # fp32 resolves L ~ 1e4 only to ~1e-3, so the bound scales with |L| here.
    parity.check_lse("geometric L", parity.f32_to_f64(L)[0, 0], eL, atol=max(1e-3, 2e-7 * eL.max()))
    ro, rL = orc.forward(*(inputs.bf16_bits_to_f64(x) for x in (qb, kb, vb)), causal, a * 16.0)
    parity.check_bf16("geometric O", parity.bf16_to_f64(o), ro)
    # V column 1 is constant 1: O must be 1 up to bf16 rounding of P.
    assert np.max(np.abs(parity.bf16_to_f64(o)[0, 0, :, 1] - 1.0)) <= 2 ** -7


def test_fwd_constant_v():
    N, d = 1000, 128
    qb, kb, _ = inputs.attention_inputs(23, 1, 4, 1, N, d)
    vb = np.broadcast_to(inputs.f32_to_bf16_bits(np.linspace(-3, 3, d, dtype=np.float32)),
                         (1, 1, N, d)).copy()
    for causal in (False, True):
        o, _ = run_fwd(qb, kb, vb, causal)
        ref = np.broadcast_to(inputs.bf16_bits_to_f64(vb)[:, :1], (1, 4, N, d))
        parity.check_bf16("O (constant V)", parity.bf16_to_f64(o), ref)


def test_fwd_gqa_equals_repeated_heads():
    qb, kb, vb = inputs.attention_inputs(24, 2, 8, 2, 777, 128)
    o1, L1 = run_fwd(qb, kb, vb, True)
    o2, L2 = run_fwd(qb, np.repeat(kb, 4, axis=1), np.repeat(vb, 4, axis=1), True)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(L1, L2)


def test_fwd_is_deterministic():
    qb, kb, vb = inputs.attention_inputs(25, 2, 4, 4, 3000, 128)
    o1, L1 = run_fwd(qb, kb, vb, True)
    o2, L2 = run_fwd(qb, kb, vb, True)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(L1, L2)


def test_fwd_large_scores_stay_finite():
    qb, kb, vb = inputs.attention_inputs(26, 1, 2, 2, 500, 64)
    q = inputs.bf16_bits_to_f32(qb) * 64.0
    qb = inputs.f32_to_bf16_bits(q)
    for causal in (False, True):
        o, L = run_fwd(qb, kb, vb, causal)
        ro, rL = orc.forward(*(inputs.bf16_bits_to_f64(x) for x in (qb, kb, vb)), causal, 0.125)
        parity.check_bf16("O (large scores)", parity.bf16_to_f64(o), ro)
        parity.check_lse("L (large scores)", parity.f32_to_f64(L), rL,
                         atol=max(1e-3, 2e-7 * np.abs(rL).max()))


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_long_sequence_sampled_rows(d, causal):
    """N = 65536 (four times the longest benchmark sequence), GQA 2:1: sampled
    rows, including the first and last rows of the sequence, against the oracle."""
    B, Hq, Hkv, N = 1, 2, 1, 65536
    log(f"[fwd] long sequence B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} causal={causal}")
    qb, kb, vb = inputs.attention_inputs(11, B, Hq, Hkv, N, d)
    o, L = run_fwd(qb, kb, vb, causal)
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(L).all())
    rows = np.array([(0, 0, 0), (0, 1, N - 1), (0, 0, N // 2), (0, 1, 255), (0, 1, 256)]
                    + [(0, int(h), int(i)) for h, i in zip(np.random.default_rng(d).integers(Hq, size=11),
                                                         np.random.default_rng(d + 1).integers(N, size=11))])
    q64, k64, v64 = (inputs.bf16_bits_to_f64(x) for x in (qb, kb, vb))
    ro, rL = orc.forward_rows(q64, k64, v64, rows, causal, 1.0 / math.sqrt(d))
    idx = torch.from_numpy(rows.astype(np.int64)).to(o.device)
    parity.check_bf16("O rows", parity.bf16_to_f64(o[idx[:, 0], idx[:, 1], idx[:, 2]]), ro)
    parity.check_lse("L rows", parity.f32_to_f64(L)[rows[:, 0], rows[:, 1], rows[:, 2]], rL)
