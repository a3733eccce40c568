"""Pins of the fp64 oracle to facts other than itself.

Each ``pin_*`` function takes a loaded oracle library and raises
AssertionError when the oracle disagrees with:

- hand-derived worked examples (``tests/golden/two_key_example.json``, and
  ``two_key_ds_example.json``, whose P and dS are not bf16-exact, for the
  working-precision roundings),
- an independent library implementation (PyTorch's CPU scaled-dot-product
  attention and autograd, float64),
- central finite differences of its own forward (for the gradients),
- closed forms (one key; zero queries; a geometric score row whose maximum
  moves at every key),
- invariants of the definition (rows of P sum to one, constant V, shifting
  keys, permuting keys, GQA equals repeated K/V heads, column sums of dV,
  causal row 0, D = rowsum(dO * O)),
- rigorous round-to-nearest-even error bounds of the working-precision
  variant (P in the forward and in dV, dS in dQ and dK), which must also be
  approached,
- for the backward from given forward outputs: PyTorch autograd (exact O, L),
  a shift of D through O, a shift of L, and the same rounding bounds,
- for block-sparse attention, PyTorch with the equivalent element mask,
  dense attention (all-ones mask) and attention over a subset of the rows
  (rows the mask empties).

The definition pinned is O = softmax(scale * Q K^T [+ causal mask]) V with
L = m + ln(l) and D = rowsum(dO o O) (FlashAttention-2 summary page,
zhaifeiyue.github.io, section 3 "Target operation" and the section 4
symbol table), GQA by shared K/V heads with dK/dV summed over the sharing
query heads (section 4 checks).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

from oracle import oracle as orc

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    assert err <= tol * scale, f"{what}: max abs err {err:.3e} > {tol:.1e} * {scale:.3g}"


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# ----------------------------------------------------------------------------
# 1. hand-derived worked example
# ----------------------------------------------------------------------------
def _golden_value(x):
    if isinstance(x, list):
        return [_golden_value(y) for y in x]
    if isinstance(x, str):
        return float(eval(x, {"__builtins__": {}}, {"ln2": math.log(2.0), "ln3": math.log(3.0),
                                                    "ln4": math.log(4.0)}))
    return float(x)


def pin_golden_two_key(lib):
    with open(os.path.join(GOLDEN, "two_key_example.json")) as f:
        g = json.load(f)
    q = np.array(_golden_value(g["Q"])).reshape(1, 1, 2, 1)
    k = np.array(_golden_value(g["K"])).reshape(1, 1, 2, 1)
    v = np.array(_golden_value(g["V"])).reshape(1, 1, 2, 1)
    do = np.array(_golden_value(g["dO"])).reshape(1, 1, 2, 1)
    for causal, key in ((False, "noncausal"), (True, "causal")):
        exp = {n: np.array(_golden_value(val)) for n, val in g[key].items()}
        o, L = orc.forward(q, k, v, causal, g["scale"], lib=lib)
        _close(o.reshape(2, 1), exp["O"], 1e-14, f"golden {key} O")
        _close(L.reshape(2), exp["L"], 1e-14, f"golden {key} L")
        dq, dk, dv, D = orc.backward(q, k, v, do, causal, g["scale"], lib=lib)
        _close(D.reshape(2), exp["D"], 1e-14, f"golden {key} D")
        _close(dq.reshape(2, 1), exp["dQ"], 1e-14, f"golden {key} dQ")
        _close(dk.reshape(2, 1), exp["dK"], 1e-14, f"golden {key} dK")
        _close(dv.reshape(2, 1), exp["dV"], 1e-14, f"golden {key} dV")


def _load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        g = json.load(f)
    arrays = [np.array(_golden_value(g[n])).reshape(1, 1, 2, 1) for n in ("Q", "K", "V", "dO")]
    return g, arrays


def pin_golden_ds_example(lib):
    """Second hand-derived example: row 1 has P = (1/3, 2/3), so P and dS are not
    bf16-exact and the working-precision backward must round them (dV from
    bf16(P), dQ and dK from bf16(dS)).  Also pins the backward from given O and L."""
    g, (q, k, v, do) = _load_golden("two_key_ds_example.json")
    for causal, key in ((False, "noncausal"), (True, "causal")):
        exp = {n: np.array(_golden_value(val)) for n, val in g[key].items()}
        wp = {n: np.array(_golden_value(val)) for n, val in g["working_precision"][key].items()}
        o, L = orc.forward(q, k, v, causal, g["scale"], lib=lib)
        _close(o.reshape(2, 1), exp["O"], 1e-14, f"ds golden {key} O")
        _close(L.reshape(2), exp["L"], 1e-14, f"ds golden {key} L")
        dq, dk, dv, D = orc.backward(q, k, v, do, causal, g["scale"], lib=lib)
        _close(D.reshape(2), exp["D"], 1e-14, f"ds golden {key} D")
        for n, a in (("dQ", dq), ("dK", dk), ("dV", dv)):
            _close(a.reshape(2, 1), exp[n], 1e-14, f"ds golden {key} {n}")
        ob, _ = orc.forward_bf16(q, k, v, causal, g["scale"], lib=lib)
        _close(ob.reshape(2, 1), wp["O"], 1e-14, f"ds golden working-precision {key} O")
        for n, a in zip(("dQ", "dK", "dV"), orc.backward_bf16(q, k, v, do, causal, g["scale"], lib=lib)):
            _close(a.reshape(2, 1), wp[n], 1e-14, f"ds golden working-precision {key} {n}")
        # The backward from given O and L: the exact forward's outputs give the exact
        # gradients, and at working precision the rounded ones.
        o_given, L_given = exp["O"].reshape(1, 1, 2, 1), exp["L"].reshape(1, 1, 2)
        for n, a in zip(("dQ", "dK", "dV"),
                        orc.backward_given(q, k, v, o_given, L_given, do, causal, g["scale"], lib=lib)):
            _close(a.reshape(2, 1), exp[n], 1e-14, f"ds golden given {key} {n}")
        for n, a in zip(("dQ", "dK", "dV"),
                        orc.backward_given(q, k, v, o_given, L_given, do, causal, g["scale"], lib=lib,
                                           working_precision=True)):
            _close(a.reshape(2, 1), wp[n], 1e-14, f"ds golden given working-precision {key} {n}")


# ----------------------------------------------------------------------------
# 2. an independent library implementation (PyTorch CPU, float64)
# ----------------------------------------------------------------------------
TORCH_CASES = [
    # (B, Hq, Hkv, N, d, causal)
    (1, 1, 1, 1, 3, False), (1, 1, 1, 1, 3, True),
    (2, 1, 1, 5, 1, False), (2, 1, 1, 5, 1, True),
    (1, 2, 1, 17, 3, False), (1, 2, 1, 17, 3, True),
    (2, 4, 2, 33, 16, False), (2, 4, 2, 33, 16, True),
    (1, 4, 1, 64, 8, True), (1, 3, 3, 40, 5, False),
]


def _torch_reference(q, k, v, causal, scale, do=None):
    import torch
    import torch.nn.functional as F
    tq = torch.tensor(q, dtype=torch.float64, requires_grad=do is not None)
    tk = torch.tensor(k, dtype=torch.float64, requires_grad=do is not None)
    tv = torch.tensor(v, dtype=torch.float64, requires_grad=do is not None)
    G = q.shape[1] // k.shape[1]
    o = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale,
                                       enable_gqa=(G > 1))
    with torch.no_grad():
        kr = tk.repeat_interleave(G, dim=1)
        s = scale * torch.matmul(tq, kr.transpose(-1, -2).contiguous())
        if causal:
            n = q.shape[2]
            s = s.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), float("-inf"))
        lse = torch.logsumexp(s, dim=-1)
    if do is None:
        return o.detach().numpy(), lse.numpy()
    o.backward(torch.tensor(do, dtype=torch.float64))
    return (o.detach().numpy(), lse.numpy(), tq.grad.numpy(), tk.grad.numpy(),
            tv.grad.numpy())


def pin_torch_forward(lib):
    rng = np.random.default_rng(11)
    for (B, Hq, Hkv, N, d, causal) in TORCH_CASES:
        q, k, v = _rand(rng, B, Hq, N, d), _rand(rng, B, Hkv, N, d), _rand(rng, B, Hkv, N, d)
        scale = 0.7 / math.sqrt(d)
        o, L = orc.forward(q, k, v, causal, scale, lib=lib)
        to, tL = _torch_reference(q, k, v, causal, scale)
        case = f"B{B} Hq{Hq} Hkv{Hkv} N{N} d{d} causal{int(causal)}"
        _close(o, to, 1e-12, f"torch fwd O {case}")
        _close(L, tL, 1e-12, f"torch fwd L {case}")


def pin_torch_backward(lib):
    rng = np.random.default_rng(12)
    for (B, Hq, Hkv, N, d, causal) in TORCH_CASES:
        q, k, v = _rand(rng, B, Hq, N, d), _rand(rng, B, Hkv, N, d), _rand(rng, B, Hkv, N, d)
        do = _rand(rng, B, Hq, N, d)
        scale = 1.3 / math.sqrt(d)
        dq, dk, dv, D = orc.backward(q, k, v, do, causal, scale, lib=lib)
        to, _, tdq, tdk, tdv = _torch_reference(q, k, v, causal, scale, do)
        case = f"B{B} Hq{Hq} Hkv{Hkv} N{N} d{d} causal{int(causal)}"
        _close(dq, tdq, 1e-11, f"torch dQ {case}")
        _close(dk, tdk, 1e-11, f"torch dK {case}")
        _close(dv, tdv, 1e-11, f"torch dV {case}")
        _close(D, np.sum(do * to, axis=-1), 1e-12, f"D = rowsum(dO*O) {case}")


# ----------------------------------------------------------------------------
# 3. central finite differences of the oracle's own forward
# ----------------------------------------------------------------------------
def pin_finite_differences(lib):
    rng = np.random.default_rng(13)
    h = 1e-6
    for (B, Hq, Hkv, N, d, causal) in [(1, 1, 1, 6, 3, False), (1, 1, 1, 7, 4, True),
                                       (1, 2, 1, 5, 2, True), (1, 2, 1, 8, 3, False)]:
        q, k, v = _rand(rng, B, Hq, N, d), _rand(rng, B, Hkv, N, d), _rand(rng, B, Hkv, N, d)
        do = _rand(rng, B, Hq, N, d)
        scale = 0.9

        def f(q_, k_, v_):
            o, _ = orc.forward(q_, k_, v_, causal, scale, lib=lib)
            return float(np.sum(do * o))

        dq, dk, dv, _ = orc.backward(q, k, v, do, causal, scale, lib=lib)
        for name, x, g in (("dQ", q, dq), ("dK", k, dk), ("dV", v, dv)):
            fd = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp = x.copy(); xp[idx] += h
                xm = x.copy(); xm[idx] -= h
                args_p = {"dQ": (xp, k, v), "dK": (q, xp, v), "dV": (q, k, xp)}[name]
                args_m = {"dQ": (xm, k, v), "dK": (q, xm, v), "dV": (q, k, xm)}[name]
                fd[idx] = (f(*args_p) - f(*args_m)) / (2 * h)
            err = np.max(np.abs(fd - g))
            ref = max(1e-3, np.max(np.abs(g)))
            assert err <= 1e-7 * ref * 10, f"finite differences {name} N{N} causal{causal}: {err:.3e}"


# ----------------------------------------------------------------------------
# 4. closed forms
# ----------------------------------------------------------------------------
def geometric_expected(N, a, causal):
    """Closed forms for Q_i = (1,0..), K_j = (j,0..) scaled so S_ij = a*j, V_j = (j/256, 0..).

    Row i sums over j <= n with n = i (causal) or N-1.  With r = exp(-a):
    L_i = a*n + ln((1 - r^(n+1)) / (1 - r)) and O_i0 = (n - sum_k k r^k / sum_k r^k) / 256,
    using sum_{k=0}^{n} r^k = (1-r^(n+1))/(1-r) and
    sum_{k=0}^{n} k r^k = r (1 - (n+1) r^n + n r^(n+1)) / (1-r)^2.
    """
    r = math.exp(-a)
    L = np.empty(N)
    O0 = np.empty(N)
    for i in range(N):
        n = i if causal else N - 1
        s0 = (1 - r ** (n + 1)) / (1 - r)
        s1 = r * (1 - (n + 1) * r ** n + n * r ** (n + 1)) / (1 - r) ** 2
        L[i] = a * n + math.log(s0)
        O0[i] = (n - s1 / s0) / 256.0
    return L, O0


def pin_closed_forms(lib):
    rng = np.random.default_rng(14)
    # One key: O = V_0, L = scale * q . k_0.
    q, k, v = _rand(rng, 2, 3, 1, 5), _rand(rng, 2, 3, 1, 5), _rand(rng, 2, 3, 1, 5)
    for causal in (False, True):
        o, L = orc.forward(q, k, v, causal, 0.37, lib=lib)
        _close(o, v, 1e-15, "N=1 O")
        _close(L, 0.37 * np.sum(q * k, axis=-1), 1e-15, "N=1 L")
    # Causal row 0 sees key 0 only.
    N, d = 9, 4
    q, k, v = _rand(rng, 1, 2, N, d), _rand(rng, 1, 2, N, d), _rand(rng, 1, 2, N, d)
    o, L = orc.forward(q, k, v, True, 0.5, lib=lib)
    _close(o[:, :, 0], v[:, :, 0], 1e-15, "causal row 0 O")
    _close(L[:, :, 0], 0.5 * np.sum(q[:, :, 0] * k[:, :, 0], axis=-1), 1e-15, "causal row 0 L")
    # Zero queries: uniform weights; L = ln(count), O = mean (prefix mean if causal).
    q = np.zeros((1, 2, N, d))
    o, L = orc.forward(q, k, v, False, 1.0, lib=lib)
    _close(L, np.full((1, 2, N), math.log(N)), 1e-14, "Q=0 L")
    _close(o, np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape), 1e-14, "Q=0 O")
    o, L = orc.forward(q, k, v, True, 1.0, lib=lib)
    cnt = np.arange(1, N + 1, dtype=np.float64)
    _close(L, np.broadcast_to(np.log(cnt), L.shape), 1e-14, "Q=0 causal L")
    _close(o, np.cumsum(v, axis=2) / cnt[None, None, :, None], 1e-14, "Q=0 causal O")
    # Geometric row: S_ij = a*j grows along the row, so the row maximum moves at every key.
    for N, a, causal in ((40, 0.3, True), (40, 0.3, False), (257, 0.05, True), (100, 2.5, True)):
        d = 3
        q = np.zeros((1, 1, N, d)); q[..., 0] = 2.0 ** -4
        k = np.zeros((1, 1, N, d)); k[0, 0, :, 0] = np.arange(N)
        v = np.zeros((1, 1, N, d)); v[0, 0, :, 0] = np.arange(N) / 256.0
        scale = a * 16.0
        o, L = orc.forward(q, k, v, causal, scale, lib=lib)
        eL, eO = geometric_expected(N, a, causal)
        _close(L[0, 0], eL, 1e-13, f"geometric L N{N} a{a} causal{causal}")
        _close(o[0, 0, :, 0], eO, 1e-13, f"geometric O N{N} a{a} causal{causal}")
        _close(o[0, 0, :, 1:], np.zeros((N, d - 1)), 0, "geometric O zero columns")


# ----------------------------------------------------------------------------
# 5. invariants
# ----------------------------------------------------------------------------
def pin_invariants(lib):
    rng = np.random.default_rng(15)
    B, Hq, Hkv, N, d = 2, 4, 2, 23, 6
    G = Hq // Hkv
    q, k, v = _rand(rng, B, Hq, N, d), _rand(rng, B, Hkv, N, d), _rand(rng, B, Hkv, N, d)
    do = _rand(rng, B, Hq, N, d)
    scale = 0.8
    kr = np.repeat(k, G, axis=1)
    vr = np.repeat(v, G, axis=1)
    for causal in (False, True):
        tag = f"causal{int(causal)}"
        o, L = orc.forward(q, k, v, causal, scale, lib=lib)
        # Rows of P = exp(S - L) sum to one (S recomputed here, with the mask).
        s = scale * np.einsum("bhid,bhjd->bhij", q, kr)
        if causal:
            s = np.where(np.triu(np.ones((N, N), bool), 1), -np.inf, s)
        _close(np.sum(np.exp(s - L[..., None]), axis=-1), np.ones_like(L), 1e-13, f"rowsum P {tag}")
        # Constant V gives constant O.
        vc = np.broadcast_to(rng.standard_normal((1, 1, 1, d)), v.shape).copy()
        oc, _ = orc.forward(q, k, vc, causal, scale, lib=lib)
        _close(oc, np.broadcast_to(vc[:, :1, :1], oc.shape), 1e-13, f"constant V {tag}")
        # Shifting every key by u leaves O unchanged and shifts L_i by scale * q_i . u.
        u = rng.standard_normal(d)
        os_, Ls = orc.forward(q, k + u, v, causal, scale, lib=lib)
        _close(os_, o, 1e-12, f"key shift O {tag}")
        _close(Ls, L + scale * np.einsum("bhid,d->bhi", q, u), 1e-12, f"key shift L {tag}")
        # GQA equals the same computation on repeated K/V heads.
        o2, L2 = orc.forward(q, kr, vr, causal, scale, lib=lib)
        _close(o, o2, 1e-15, f"GQA forward {tag}")
        _close(L, L2, 1e-15, f"GQA L {tag}")
        dq, dk, dv, D = orc.backward(q, k, v, do, causal, scale, lib=lib)
        dq2, dk2, dv2, D2 = orc.backward(q, kr, vr, do, causal, scale, lib=lib)
        _close(dq, dq2, 1e-14, f"GQA dQ {tag}")
        _close(dk, dk2.reshape(B, Hkv, G, N, d).sum(axis=2), 1e-13, f"GQA dK {tag}")
        _close(dv, dv2.reshape(B, Hkv, G, N, d).sum(axis=2), 1e-13, f"GQA dV {tag}")
        # D = rowsum(dO o O).
        _close(D, np.sum(do * o, axis=-1), 1e-13, f"D identity {tag}")
        # Rows of P sum to one, so sum_j dV_j = sum_i dO_i (per KV head).
        _close(dv.sum(axis=2), do.reshape(B, Hkv, G, N, d).sum(axis=(2, 3)), 1e-12,
               f"sum dV {tag}")
        # Rows of dS sum to zero, so sum_j dK_j = 0 (per KV head).
        _close(dk.sum(axis=2), np.zeros((B, Hkv, d)), 1e-12, f"sum dK {tag}")
        # Constant V: O does not depend on Q or K, so dQ = dK = 0 and dV_j = sum_i P_ij dO_i.
        dqc, dkc, dvc, _ = orc.backward(q, k, vc, do, causal, scale, lib=lib)
        _close(dqc, np.zeros_like(dqc), 1e-13, f"constant V dQ {tag}")
        _close(dkc, np.zeros_like(dkc), 1e-13, f"constant V dK {tag}")
        if causal:
            _close(dq[:, :, 0], np.zeros((B, Hq, d)), 0, "causal dQ row 0")
    # Non-causal: permuting keys and values together changes nothing.
    perm = rng.permutation(N)
    o, L = orc.forward(q, k, v, False, scale, lib=lib)
    op, Lp = orc.forward(q, k[:, :, perm], v[:, :, perm], False, scale, lib=lib)
    _close(op, o, 1e-13, "key permutation O")
    _close(Lp, L, 1e-13, "key permutation L")
    # Large scores: exact max subtraction keeps everything finite.
    o, L = orc.forward(q * 64, k, v, True, scale, lib=lib)
    to, tL = _torch_reference(q * 64, k, v, True, scale)
    _close(o, to, 1e-12, "large scores O")
    _close(L, tL, 1e-12, "large scores L")


def pin_sampled_entry_points(lib):
    """The per-row forward and per-head backward agree with the full versions."""
    rng = np.random.default_rng(16)
    B, Hq, Hkv, N, d = 2, 4, 2, 19, 5
    q, k, v = _rand(rng, B, Hq, N, d), _rand(rng, B, Hkv, N, d), _rand(rng, B, Hkv, N, d)
    do = _rand(rng, B, Hq, N, d)
    for causal in (False, True):
        o, L = orc.forward(q, k, v, causal, 0.6, lib=lib)
        rows = np.array([[0, 0, 0], [1, 3, 18], [0, 2, 7], [1, 1, 11]])
        orow, Lrow = orc.forward_rows(q, k, v, rows, causal, 0.6, lib=lib)
        _close(orow, o[rows[:, 0], rows[:, 1], rows[:, 2]], 0, "forward_rows O")
        _close(Lrow, L[rows[:, 0], rows[:, 1], rows[:, 2]], 0, "forward_rows L")
        dq, dk, dv, D = orc.backward(q, k, v, do, causal, 0.6, lib=lib)
        hdq, hdk, hdv, hL, hD = orc.backward_head(q, k, v, do, 1, 1, causal, 0.6, lib=lib)
        _close(hdq, dq[1, 2:4], 0, "backward_head dQ")
        _close(hdk, dk[1, 1], 0, "backward_head dK")
        _close(hdv, dv[1, 1], 0, "backward_head dV")
        _close(hL, L[1, 2:4], 0, "backward_head L")
        _close(hD, D[1, 2:4], 0, "backward_head D")


# ----------------------------------------------------------------------------
# 6. the working-precision variant (bf16 P, O and dS at the method's rounding points)
# ----------------------------------------------------------------------------
U_BF16 = 2.0 ** -8 + 2.0 ** -23     # RNE to 8 significant bits, after a first rounding to fp32


def pin_working_precision(lib):
    # The two-key example (hand-derived working-precision values in the golden file):
    # the forward rounds the unnormalized exp(S - rowmax) = 1/3 of row 1; every
    # backward rounding point holds a bf16-exact value.
    with open(os.path.join(GOLDEN, "two_key_example.json")) as f:
        g = json.load(f)
    q = np.array(_golden_value(g["Q"])).reshape(1, 1, 2, 1)
    k = np.array(_golden_value(g["K"])).reshape(1, 1, 2, 1)
    v = np.array(_golden_value(g["V"])).reshape(1, 1, 2, 1)
    do = np.array(_golden_value(g["dO"])).reshape(1, 1, 2, 1)
    for causal, key in ((False, "noncausal"), (True, "causal")):
        exp = {n: np.array(_golden_value(val)) for n, val in g[key].items()}
        o, L = orc.forward_bf16(q, k, v, causal, g["scale"], lib=lib)
        wp = np.array([[float(eval(str(x), {"__builtins__": {}})) for x in r]
                       for r in g["working_precision"][key]["O"]])
        _close(o.reshape(2, 1), wp, 1e-14, f"bf16 golden {key} O")
        _close(L.reshape(2), exp["L"], 1e-14, f"bf16 golden {key} L")
        dq, dk, dv = orc.backward_bf16(q, k, v, do, causal, g["scale"], lib=lib)
        _close(dq.reshape(2, 1), exp["dQ"], 1e-14, f"bf16 golden {key} dQ")
        _close(dk.reshape(2, 1), exp["dK"], 1e-14, f"bf16 golden {key} dK")
        _close(dv.reshape(2, 1), exp["dV"], 1e-14, f"bf16 golden {key} dV")
    # Rigorous first-order bounds of the roundings, which must also be approached
    # (so the rounding really happens, to 8 significant bits).
    rng = np.random.default_rng(17)
    B, Hq, Hkv, N, d = 1, 2, 1, 60, 8
    q, k, v = _rand(rng, B, Hq, N, d), _rand(rng, B, Hkv, N, d), _rand(rng, B, Hkv, N, d)
    do = _rand(rng, B, Hq, N, d)
    scale = 0.9
    kr, vr = np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1)
    for causal in (False, True):
        s = scale * np.einsum("bhid,bhjd->bhij", q, kr)
        if causal:
            s = np.where(np.triu(np.ones((N, N), bool), 1), -np.inf, s)
        p = np.exp(s - s.max(-1, keepdims=True))
        l = p.sum(-1, keepdims=True)
        o_ex, L_ex = orc.forward(q, k, v, causal, scale, lib=lib)
        o_b, L_b = orc.forward_bf16(q, k, v, causal, scale, lib=lib)
        _close(L_b, L_ex, 1e-13, "bf16 forward L is unrounded")
        bound = U_BF16 * np.einsum("bhij,bhjd->bhid", p, np.abs(vr)) / l
        ratio = np.abs(o_b - o_ex) / np.maximum(bound, 1e-300)
        assert ratio.max() <= 1.0 + 1e-9, f"forward rounding above its bound: {ratio.max()}"
        assert ratio.max() >= 0.25, f"forward rounding far below its bound: {ratio.max()}"
        P = np.exp(s - L_ex[..., None])
        _, _, dv_ex, _ = orc.backward(q, k, v, do, causal, scale, lib=lib)
        _, _, dv_b = orc.backward_bf16(q, k, v, do, causal, scale, lib=lib)
        bound = U_BF16 * np.einsum("bhij,bhid->bhjd", P, np.abs(do)).reshape(B, Hkv, 2, N, d).sum(2)
        ratio = np.abs(dv_b - dv_ex) / np.maximum(bound, 1e-300)
        assert ratio.max() <= 1.0 + 1e-9, f"dV rounding above its bound: {ratio.max()}"
        assert ratio.max() >= 0.25, f"dV rounding far below its bound: {ratio.max()}"
        # D is formed from the stored (bf16) O of the working-precision forward.
        dq_b, dk_b, _, D_b = orc.backward_bf16(q, k, v, do, causal, scale, lib=lib, return_d=True)
        # dQ and dK: the products take bf16(dS) with dS = P o (dP - D) at that D; each
        # element is off by at most U * scale * sum |dS| |K| (|Q|) from the unrounded
        # products, and must come close to that bound.
        dP = np.einsum("bhid,bhjd->bhij", do, vr)
        dS = P * (dP - D_b[..., None])
        dq_u = scale * np.einsum("bhij,bhjd->bhid", dS, kr)
        dk_u = scale * np.einsum("bhij,bhid->bhjd", dS, q).reshape(B, Hkv, 2, N, d).sum(2)
        for name, got, unr, bound in (
                ("dQ", dq_b, dq_u, U_BF16 * scale * np.einsum("bhij,bhjd->bhid", np.abs(dS), np.abs(kr))),
                ("dK", dk_b, dk_u, U_BF16 * scale * np.einsum("bhij,bhid->bhjd", np.abs(dS), np.abs(q))
                 .reshape(B, Hkv, 2, N, d).sum(2))):
            ratio = np.abs(got - unr) / np.maximum(bound, 1e-300)
            assert ratio.max() <= 1.0 + 1e-9, f"{name} dS rounding above its bound: {ratio.max()}"
            assert ratio.max() >= 0.25, f"{name} dS rounding far below its bound: {ratio.max()}"
        o_stored = o_b.astype(np.float32).view(np.uint32).astype(np.uint64)
        o_stored = (((o_stored + 0x7FFF + ((o_stored >> 16) & 1)) >> 16) << 16).astype(np.uint32)
        o_stored = o_stored.view(np.float32).astype(np.float64)
        _close(D_b, np.sum(do * o_stored, axis=-1), 1e-13, "bf16 D from the stored O")
        assert np.max(np.abs(D_b - np.sum(do * o_b, axis=-1))) > 1e-6, "D ignores the O rounding"
        # The one-head entry point agrees with the full one.
        dq_b, dk_b, dv_b2 = orc.backward_bf16(q, k, v, do, causal, scale, lib=lib)
        hq_, hk_, hv_ = orc.backward_bf16_head(q, k, v, do, 0, 0, causal, scale, lib=lib)
        _close(hq_, dq_b[0], 0, "bf16 head dQ")
        _close(hk_, dk_b[0, 0], 0, "bf16 head dK")
        _close(hv_, dv_b2[0, 0], 0, "bf16 head dV")


# ----------------------------------------------------------------------------
# 6b. the backward from given forward outputs (O, L)
# ----------------------------------------------------------------------------
def pin_backward_given(lib):
    """P is rebuilt from the given L and D is formed from the given O:
    - with the exact forward's O and L it equals PyTorch's fp64 autograd;
    - moving O_i along dO_i so that D_i shifts by c_i leaves dV unchanged, leaves dQ_i
      unchanged where c_i = 0, and (rows of P summing to one) gives
      sum_j dS_ij = -c_i, so sum_j dK_j = -scale * sum_i c_i Q_i per K/V head;
    - raising every L_i by c scales P, hence dV, by exp(-c);
    - at working precision, each gradient is within the RNE bound of its rounded
      operand (P for dV, dS for dQ and dK) of the exact one and comes close to it."""
    rng = np.random.default_rng(18)
    B, Hq, Hkv, N, d = 2, 4, 2, 29, 6
    G = Hq // Hkv
    q, k, v = _rand(rng, B, Hq, N, d), _rand(rng, B, Hkv, N, d), _rand(rng, B, Hkv, N, d)
    do = _rand(rng, B, Hq, N, d)
    scale = 0.85
    kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    for causal in (False, True):
        tag = f"causal{int(causal)}"
        o, L = orc.forward(q, k, v, causal, scale, lib=lib)
        dq, dk, dv = orc.backward_given(q, k, v, o, L, do, causal, scale, lib=lib)
        to, _, tdq, tdk, tdv = _torch_reference(q, k, v, causal, scale, do)
        _close(dq, tdq, 1e-11, f"given dQ vs torch {tag}")
        _close(dk, tdk, 1e-11, f"given dK vs torch {tag}")
        _close(dv, tdv, 1e-11, f"given dV vs torch {tag}")
        c = rng.standard_normal((B, Hq, N))
        c[:, :, ::3] = 0.0
        o2 = o + c[..., None] * do / np.sum(do * do, axis=-1, keepdims=True)
        dq2, dk2, dv2 = orc.backward_given(q, k, v, o2, L, do, causal, scale, lib=lib)
        _close(dv2, dv, 1e-13, f"given D shift leaves dV {tag}")
        _close(dq2[:, :, ::3], dq[:, :, ::3], 1e-12, f"given D shift leaves dQ of unshifted rows {tag}")
        assert np.max(np.abs(dq2 - dq)) > 1e-3, f"given O ignored in dQ {tag}"
        want = -scale * np.einsum("bhi,bhid->bhd", c, q).reshape(B, Hkv, G, d).sum(2)
        _close(dk2.sum(axis=2), want, 1e-12, f"given D shift: column sum of dK {tag}")
        _close(dk.sum(axis=2), np.zeros((B, Hkv, d)), 1e-12, f"given exact: column sum of dK {tag}")
        _, _, dv3 = orc.backward_given(q, k, v, o, L + 0.4, do, causal, scale, lib=lib)
        _close(dv3, math.exp(-0.4) * dv, 1e-13, f"given L shift scales dV {tag}")
        # Working precision from the same given O and L.
        s = scale * np.einsum("bhid,bhjd->bhij", q, kr)
        if causal:
            s = np.where(np.triu(np.ones((N, N), bool), 1), -np.inf, s)
        P = np.exp(s - L[..., None])
        dS = P * (np.einsum("bhid,bhjd->bhij", do, vr) - np.sum(do * o, axis=-1)[..., None])
        wq, wk, wv = orc.backward_given(q, k, v, o, L, do, causal, scale, lib=lib, working_precision=True)
        sum_g = lambda x: x.reshape(B, Hkv, G, N, d).sum(2)
        for name, got, ex, bound in (
                ("dV", wv, dv, U_BF16 * sum_g(np.einsum("bhij,bhid->bhjd", P, np.abs(do)))),
                ("dQ", wq, dq, U_BF16 * scale * np.einsum("bhij,bhjd->bhid", np.abs(dS), np.abs(kr))),
                ("dK", wk, dk, U_BF16 * scale * sum_g(np.einsum("bhij,bhid->bhjd", np.abs(dS), np.abs(q))))):
            ratio = np.abs(got - ex) / np.maximum(bound, 1e-300)
            assert ratio.max() <= 1.0 + 1e-9, f"given working-precision {name} above its bound {tag}: {ratio.max()}"
            assert ratio.max() >= 0.25, f"given working-precision {name} far below its bound {tag}: {ratio.max()}"


# ----------------------------------------------------------------------------
# 7. block-sparse attention
# ----------------------------------------------------------------------------
def _element_mask(block_mask, N, causal):
    """Allowed (query, key) pairs: the block mask expanded to elements, and the causal mask."""
    bs = orc.SPARSE_BLOCK
    idx = np.arange(N) // bs
    allowed = np.asarray(block_mask, dtype=bool)[idx[:, None], idx[None, :]]
    if causal:
        allowed &= np.tril(np.ones((N, N), dtype=bool))
    return allowed


def _torch_masked(q, k, v, do, allowed, scale):
    """PyTorch CPU float64 attention with an explicit boolean mask, and its gradients."""
    import torch
    import torch.nn.functional as F
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    G = q.shape[1] // k.shape[1]
    m = torch.tensor(allowed)
    o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=m, scale=scale, enable_gqa=(G > 1))
    with torch.no_grad():
        kr = tk.repeat_interleave(G, dim=1)
        sc = scale * torch.matmul(tq, kr.transpose(-1, -2).contiguous())
        lse = torch.logsumexp(sc.masked_fill(~m, float("-inf")), dim=-1)
    o.backward(torch.tensor(do, dtype=torch.float64))
    return (o.detach().numpy(), lse.numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy())


def pin_block_sparse(lib):
    """Block masks against PyTorch with the equivalent element mask (asymmetric masks, so a
    transposed or ignored mask fails), all-ones masks against dense attention, and rows the
    mask empties (L = -inf, O = 0, no gradient) against attention over the other rows."""
    rng = np.random.default_rng(17)
    B, Hq, Hkv, N, d = 1, 2, 1, 300, 4          # 3 x 3 blocks, the last one ragged
    q, k, v = _rand(rng, B, Hq, N, d), _rand(rng, B, Hkv, N, d), _rand(rng, B, Hkv, N, d)
    do = _rand(rng, B, Hq, N, d)
    scale = 0.8
    masks = {
        "lower-left": np.array([[1, 0, 0], [1, 1, 0], [0, 1, 1]]),
        "upper": np.array([[0, 1, 1], [0, 0, 1], [1, 0, 0]]),
        "column 0": np.array([[1, 0, 0], [1, 0, 0], [1, 0, 0]]),
    }
    for name, bm in masks.items():
        for causal in (False, True):
            allowed = _element_mask(bm, N, causal)
            if not allowed.any(axis=1).all():
                continue                         # rows with no key: checked below
            case = f"{name} causal{int(causal)}"
            o, L = orc.forward(q, k, v, causal, scale, lib=lib, block_mask=bm)
            dq, dk, dv, D = orc.backward(q, k, v, do, causal, scale, lib=lib, block_mask=bm)
            to, tL, tdq, tdk, tdv = _torch_masked(q, k, v, do, allowed, scale)
            _close(o, to, 1e-12, f"block-sparse O {case}")
            _close(L, tL, 1e-12, f"block-sparse L {case}")
            _close(dq, tdq, 1e-11, f"block-sparse dQ {case}")
            _close(dk, tdk, 1e-11, f"block-sparse dK {case}")
            _close(dv, tdv, 1e-11, f"block-sparse dV {case}")
            _close(D, np.sum(do * to, axis=-1), 1e-12, f"block-sparse D {case}")

    ones = np.ones((3, 3))
    for causal in (False, True):
        o, L = orc.forward(q, k, v, causal, scale, lib=lib, block_mask=ones)
        o0, L0 = orc.forward(q, k, v, causal, scale, lib=lib)
        _close(o, o0, 0, "all-ones block mask O")
        _close(L, L0, 0, "all-ones block mask L")
        g = orc.backward(q, k, v, do, causal, scale, lib=lib, block_mask=ones)
        g0 = orc.backward(q, k, v, do, causal, scale, lib=lib)
        for a, b_, n in zip(g, g0, ("dQ", "dK", "dV", "D")):
            _close(a, b_, 0, f"all-ones block mask {n}")

    # Query block 1 (rows 128..255) masked entirely; causal too, so that block 0
    # attends only to itself.
    bm = np.array([[1, 0, 1], [0, 0, 0], [1, 1, 1]])
    for causal in (False, True):
        case = f"empty query block causal{int(causal)}"
        o, L = orc.forward(q, k, v, causal, scale, lib=lib, block_mask=bm)
        dq, dk, dv, D = orc.backward(q, k, v, do, causal, scale, lib=lib, block_mask=bm)
        empty = slice(128, 256)
        assert np.all(L[:, :, empty] == -np.inf), f"{case}: L of masked rows"
        assert np.all(o[:, :, empty] == 0.0), f"{case}: O of masked rows"
        assert np.all(dq[:, :, empty] == 0.0), f"{case}: dQ of masked rows"
        assert np.all(D[:, :, empty] == 0.0), f"{case}: D of masked rows"
        keep = np.r_[0:128, 256:N]
        allowed = _element_mask(bm, N, causal)[keep]
        to, tL, tdq, tdk, tdv = _torch_masked(q[:, :, keep], k, v, do[:, :, keep], allowed, scale)
        _close(o[:, :, keep], to, 1e-12, f"{case}: O of the other rows")
        _close(L[:, :, keep], tL, 1e-12, f"{case}: L of the other rows")
        _close(dq[:, :, keep], tdq, 1e-11, f"{case}: dQ of the other rows")
        _close(dk, tdk, 1e-11, f"{case}: dK")
        _close(dv, tdv, 1e-11, f"{case}: dV")
        # The working-precision variants: the same empty rows, and within bf16
        # rounding of the exact values elsewhere.
        ob, Lb = orc.forward_bf16(q, k, v, causal, scale, lib=lib, block_mask=bm)
        assert np.all(Lb[:, :, empty] == -np.inf) and np.all(ob[:, :, empty] == 0.0), \
            f"{case}: working-precision forward of masked rows"
        _close(ob[:, :, keep], o[:, :, keep], 2e-2, f"{case}: working-precision O")
        wq, wk, wv = orc.backward_bf16(q, k, v, do, causal, scale, lib=lib, block_mask=bm)
        assert np.all(wq[:, :, empty] == 0.0), f"{case}: working-precision dQ of masked rows"
        _close(wq, dq, 5e-2, f"{case}: working-precision dQ")
        _close(wk, dk, 5e-2, f"{case}: working-precision dK")
        _close(wv, dv, 5e-2, f"{case}: working-precision dV")
        # Row and head entry points agree with the full ones.
        rows = np.array([[0, 1, 5], [0, 0, 130], [0, 1, 299]])
        orow, Lrow = orc.forward_rows(q, k, v, rows, causal, scale, lib=lib, block_mask=bm)
        assert Lrow[1] == -np.inf and np.all(orow[1] == 0.0), f"{case}: forward_rows masked row"
        _close(orow[[0, 2]], o[0, rows[[0, 2], 1], rows[[0, 2], 2]], 0, f"{case}: forward_rows")
        hq_, hk_, hv_, _, _ = orc.backward_head(q, k, v, do, 0, 0, causal, scale, lib=lib,
                                                block_mask=bm)
        _close(hq_, dq[0], 0, f"{case}: backward_head dQ")
        _close(hk_, dk[0, 0], 0, f"{case}: backward_head dK")
        bq_, bk_, bv_ = orc.backward_bf16_head(q, k, v, do, 0, 0, causal, scale, lib=lib,
                                               block_mask=bm)
        _close(bq_, wq[0], 0, f"{case}: backward_bf16_head dQ")
        _close(bv_, wv[0, 0], 0, f"{case}: backward_bf16_head dV")


ALL_PINS = [pin_golden_two_key, pin_golden_ds_example, pin_torch_forward, pin_torch_backward,
            pin_finite_differences, pin_closed_forms, pin_invariants,
            pin_sampled_entry_points, pin_working_precision, pin_backward_given, pin_block_sparse]
