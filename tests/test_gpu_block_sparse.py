"""Block-sparse attention on the GPU against the fp64 oracle with the same block mask
(every head dim; bf16 and f16).

The mask (one byte per 128 x 128 block, shared by all batches and heads)
masks scores like the causal mask does; rows the mask leaves without any key
must come back as O = 0, L = -inf exactly, with dQ = 0.  Outputs are
pre-filled with NaN, the workspace with 0xFF, so unwritten elements fail.
An all-ones mask must reproduce the dense kernels bit for bit (same tiles,
same order, same arithmetic).
"""
import math

import numpy as np
import pytest

from exact_io_aware_26_amd import inputs
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


def to_dev(bits, fmt):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16 if fmt == "bf16" else torch.float16).to("cuda")


def to_f64(t):
    bits = t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return inputs.bf16_bits_to_f64(bits) if t.dtype == torch.bfloat16 else inputs.f16_bits_to_f64(bits)


def run(qb, kb, vb, dob, mask, causal, scale=None, fmt="bf16"):
    from exact_io_aware_26_amd import fa2
    q, k, v, do = (to_dev(x, fmt) for x in (qb, kb, vb, dob))
    bm = torch.from_numpy(mask).to(q.device)
    out = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=q.device)
    o, L = fa2.forward_block_sparse(q, k, v, bm, causal=causal, scale=scale, out=out, lse=lse)
    nbytes = fa2.workspace_bytes(*q.shape[:2], k.shape[1], *q.shape[2:])
    ws = torch.full((max(nbytes, 1),), 0xFF, dtype=torch.uint8, device=q.device)
    grads = tuple(torch.full_like(t, float("nan")) for t in (q, k, v))
    dq, dk, dv = fa2.backward_block_sparse(q, k, v, o, L, do, bm, causal=causal, scale=scale,
                                           workspace=ws, grads=grads)
    torch.cuda.synchronize()
    return o, L, dq, dk, dv


def check_case(seed, B, Hq, Hkv, N, d, causal, kind, backward=True, fmt="bf16"):
    mask = inputs.block_mask(kind, N, seed=seed)
    log(f"[sparse] seed={seed} B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} causal={causal} mask={kind} "
        f"({int(mask.sum())}/{mask.size} blocks) {fmt}")
    qb, kb, vb, dob = inputs.attention_inputs(seed, B, Hq, Hkv, N, d, with_grad=True, fmt=fmt)
    o, L, dq, dk, dv = run(qb, kb, vb, dob, mask, causal, fmt=fmt)
    widen = inputs.bf16_bits_to_f64 if fmt == "bf16" else inputs.f16_bits_to_f64
    q64, k64, v64, do64 = (widen(x) for x in (qb, kb, vb, dob))
    sc = 1.0 / math.sqrt(d)
    ro, rL = orc.forward(q64, k64, v64, causal, sc, block_mask=mask)
    go, gL = to_f64(o), parity.f32_to_f64(L)
    empty = np.isneginf(rL)
    # Rows without any key: exactly O = 0 and L = -inf.
    assert np.array_equal(np.isneginf(gL), empty), "rows with L = -inf differ from the oracle's"
    assert np.all(go[empty] == 0.0), "O of rows without any key must be 0"
    parity.check_bf16("O", go[~empty], ro[~empty])
    parity.check_lse("L", gL[~empty], rL[~empty])
    if not backward:
        return
    rdq, rdk, rdv, _ = orc.backward(q64, k64, v64, do64, causal, sc, block_mask=mask)
    gdq = to_f64(dq)
    assert np.all(gdq[empty] == 0.0), "dQ of rows without any key must be 0"
    if fmt == "f16":
        # The f16 path: stated gates (no working-precision widening).
        parity.check_bf16("dQ (f16)", gdq, rdq)
        parity.check_bf16("dK (f16)", to_f64(dk), rdk)
        parity.check_bf16("dV (f16)", to_f64(dv), rdv)
        return
    wdq, wdk, wdv = orc.backward_bf16(q64, k64, v64, do64, causal, sc, block_mask=mask)
    parity.check_bf16("dQ", gdq, rdq, working=wdq)
    parity.check_bf16("dK", to_f64(dk), rdk, working=wdk)
    parity.check_bf16("dV", to_f64(dv), rdv, working=wdv)


KINDS = ("random", "local_global", "diagonal", "column0", "strided", "ones", "zeros")
CASES = []
for i, N in enumerate((1, 100, 128, 129, 255, 300, 513, 700)):
    for d in (64, 128, 256):
        for causal in (False, True):
            kind = KINDS[(i + d // 64 + causal) % len(KINDS)]
            heads = [(1, 1), (4, 2), (2, 2), (4, 1)][(i + causal) % 4]
            CASES.append((1 + i % 2, heads[0], heads[1], N, d, causal, kind))


@pytest.mark.parametrize("B,Hq,Hkv,N,d,causal,kind", CASES)
def test_block_sparse_small(B, Hq, Hkv, N, d, causal, kind):
    check_case(400 + N + d, B, Hq, Hkv, N, d, causal, kind)


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("causal", [False, True])
def test_block_sparse_mask_kinds(kind, causal):
    check_case(21, 1, 2, 1, 1100, 128, causal, kind)


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("causal", [False, True])
def test_block_sparse_mask_kinds_d256(kind, causal):
    check_case(22, 1, 4, 2, 1100, 256, causal, kind)


F16_CASES = [(1, 2, 1, 300, 64, True, "random"), (2, 4, 2, 700, 128, False, "local_global"),
             (1, 4, 1, 1100, 128, True, "strided"), (1, 2, 2, 513, 256, True, "random"),
             (1, 2, 1, 1024, 256, False, "diagonal"), (1, 2, 1, 129, 64, False, "zeros")]


@pytest.mark.parametrize("B,Hq,Hkv,N,d,causal,kind", F16_CASES)
def test_block_sparse_f16(B, Hq, Hkv, N, d, causal, kind):
    """The binary16 entry points (fa2_fwd_block_sparse_f16, fa2_bwd_block_sparse_f16)."""
    check_case(600 + N + d, B, Hq, Hkv, N, d, causal, kind, fmt="f16")


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_block_sparse_random_multi_tile(d, causal):
    # Random masks differ between the two 128-row mask blocks of a 256-row
    # workgroup, so most key tiles are needed by one of them only.
    for seed in (1, 2, 3):
        check_case(seed, 1, 2, 2, 2048, d, causal, "random")


def test_block_sparse_all_ones_is_dense_bitwise():
    from exact_io_aware_26_amd import fa2
    for (N, d, causal, fmt) in ((1000, 128, True, "bf16"), (777, 64, False, "bf16"), (2048, 128, False, "bf16"),
                                (300, 64, True, "bf16"), (1000, 256, True, "bf16"), (333, 256, False, "bf16"),
                                (700, 128, True, "f16"), (515, 256, False, "f16")):
        log(f"[sparse] all-ones vs dense N={N} d={d} causal={causal} {fmt}")
        qb, kb, vb, dob = inputs.attention_inputs(77 + N, 2, 4, 2, N, d, with_grad=True, fmt=fmt)
        mask = inputs.block_mask("ones", N)
        o, L, dq, dk, dv = run(qb, kb, vb, dob, mask, causal, fmt=fmt)
        q, k, v, do = (to_dev(x, fmt) for x in (qb, kb, vb, dob))
        o2, L2 = fa2.forward(q, k, v, causal=causal)
        dq2, dk2, dv2 = fa2.backward(q, k, v, o2, L2, do, causal=causal)
        torch.cuda.synchronize()
        for name, a, b in (("O", o, o2), ("L", L, L2), ("dQ", dq, dq2), ("dK", dk, dk2), ("dV", dv, dv2)):
            assert torch.equal(a, b), f"{name}: all-ones block-sparse differs from dense"


def test_block_sparse_large_sampled_rows():
    """B2 H8 N8192 d128 causal with a sliding-window + global mask: every element finite,
    sampled rows of O and L against the oracle, one K/V head's gradients at N = 2048."""
    from exact_io_aware_26_amd import fa2
    B, Hq, Hkv, N, d = 2, 8, 8, 8192, 128
    mask = inputs.block_mask("local_global", N)
    log(f"[sparse] large B={B} H={Hq} N={N} d={d} causal local_global ({int(mask.sum())} blocks)")
    qb, kb, vb, dob = inputs.attention_inputs(5, B, Hq, Hkv, N, d, with_grad=True)
    o, L, dq, dk, dv = run(qb, kb, vb, dob, mask, True)
    for name, t in (("O", o), ("dQ", dq), ("dK", dk), ("dV", dv)):
        assert bool(torch.isfinite(t).all()), f"{name} has unwritten or non-finite elements"
    assert bool(torch.isfinite(L).all())
    rng = np.random.default_rng(3)
    rows = [(0, 0, 0), (B - 1, Hq - 1, N - 1), (1, 3, 4095), (0, 5, 640)]
    rows += [(int(rng.integers(B)), int(rng.integers(Hq)), int(rng.integers(N))) for _ in range(20)]
    rows = np.array(rows)
    q64, k64, v64 = (inputs.bf16_bits_to_f64(x) for x in (qb, kb, vb))
    ro, rL = orc.forward_rows(q64, k64, v64, rows, True, 1.0 / math.sqrt(d), block_mask=mask)
    go = parity.bf16_to_f64(o)[rows[:, 0], rows[:, 1], rows[:, 2]]
    gL = parity.f32_to_f64(L)[rows[:, 0], rows[:, 1], rows[:, 2]]
    parity.check_bf16("O rows", go, ro)
    parity.check_lse("L rows", gL, rL)
    # Gradients of one head in full at N = 2048 (the oracle's backward is quadratic per head).
    check_case(6, 1, 1, 1, 2048, 128, True, "local_global")
    del fa2


@pytest.mark.parametrize("d", [64, 128, 256])
def test_block_sparse_maximum_n(d):
    """N = 262144 (the largest block-sparse N: 4096 tiles of 64 keys, the top of
    the tile lists' 12-bit index; at d = 256, 8192 tiles of 32 keys) with a
    local + global mask: sampled rows of O and L against the oracle, including
    rows of the last block; every gradient element written and finite."""
    from exact_io_aware_26_amd import fa2
    B, Hq, Hkv, N = 1, 1, 1, fa2.SPARSE_MAX_N
    mask = inputs.block_mask("local_global", N)
    log(f"[sparse] maximum N={N} d={d} causal local_global ({int(mask.sum())} blocks)")
    qb, kb, vb, dob = inputs.attention_inputs(9, B, Hq, Hkv, N, d, with_grad=True)
    o, L, dq, dk, dv = run(qb, kb, vb, dob, mask, True)
    for name, t in (("O", o), ("dQ", dq), ("dK", dk), ("dV", dv)):
        assert bool(torch.isfinite(t).all()), f"{name} has unwritten or non-finite elements"
    rng = np.random.default_rng(4)
    rows = [(0, 0, 0), (0, 0, N - 1), (0, 0, N - 129), (0, 0, 131071)]
    rows += [(0, 0, int(rng.integers(N))) for _ in range(12)]
    rows = np.array(rows)
    q64, k64, v64 = (inputs.bf16_bits_to_f64(x) for x in (qb, kb, vb))
    ro, rL = orc.forward_rows(q64, k64, v64, rows, True, 1.0 / math.sqrt(d), block_mask=mask)
    parity.check_bf16("O rows", parity.bf16_to_f64(o)[rows[:, 0], rows[:, 1], rows[:, 2]], ro)
    parity.check_lse("L rows", parity.f32_to_f64(L)[rows[:, 0], rows[:, 1], rows[:, 2]], rL)
