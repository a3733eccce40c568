"""Comparison of GPU results with the fp64 oracle, and tensor marshalling for GPU tests.

Tolerances (bf16 outputs O, dQ, dK, dV): max-abs error 1e-2 and relative L2
error 5e-3; fp32 L: max-abs 1e-3.  The max-abs gate is applied to the error
beyond the mandatory rounding of the exact value to bf16 (half a bf16 ulp of
the reference value): for |x| >= 4 a bf16 ulp is already 0.03, so no stored
bf16 value can be within 1e-2 of every exact value there.  The raw max-abs
error is reported alongside and gated as well wherever every reference
value is below 2 in magnitude (half an ulp there is at most 0.0039).

Widened gates.  The benchmark configurations are always held to the stated
gates.  A test of another shape may pass ``working=``, the oracle's result at
the method's working precision (bf16 P, stored bf16 O and bf16 dS): its gates
then become 1.5 times the error of that exact bf16 execution where this is
larger than the stated gate, but never more than a fixed ceiling (``CAP_ATOL``
for the max-abs gates, ``CAP_RL2`` for relative L2, unless the test states its
own).  Every widened gate is printed as ``[gate] ...`` with the stated and the
applied value, and appended to the file named by ``FA2_GATE_LOG`` if set.
"""
from __future__ import annotations

import os
import sys

import numpy as np

from exact_io_aware_26_amd import inputs

ATOL_BF16 = 1e-2
RL2_BF16 = 5e-3
ATOL_L = 1e-3
# Ceilings on a widened gate.  The max-abs ceiling covers the method's own
# error at the default scale (up to about 0.015 beyond rounding on small causal
# problems, through D formed from the stored bf16 O); the relative-L2 ceiling
# covers tensors of one or two rows, whose norm is tiny.
CAP_ATOL = 2e-2
CAP_RL2 = 4e-2


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def half_ulp_bf16(ref: np.ndarray) -> np.ndarray:
    a = np.abs(ref)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return np.ldexp(1.0, (e - 8).astype(np.int64))


def metrics(got: np.ndarray, ref: np.ndarray) -> dict:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    excess = np.maximum(0.0, err - half_ulp_bf16(ref))
    denom = np.linalg.norm(ref.ravel())
    return {
        "max_abs": float(err.max()) if err.size else 0.0,
        "max_abs_beyond_rounding": float(excess.max()) if err.size else 0.0,
        "rel_l2": float(np.linalg.norm((got - ref).ravel()) / denom) if denom > 0 else float(err.max(initial=0.0)),
        "ref_max": float(np.abs(ref).max()) if ref.size else 0.0,
        "finite": bool(np.all(np.isfinite(got))),
    }


def round_bf16(x: np.ndarray) -> np.ndarray:
    return inputs.bf16_bits_to_f64(inputs.f32_to_bf16_bits(np.asarray(x, dtype=np.float32)))


def _log_gate(name: str, m: dict, stated: tuple, applied: tuple) -> None:
    w = m["working_precision"]
    test = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
    line = (f"[gate] {test} {name}: beyond-rounding stated {stated[0]:.1e} applied {applied[0]:.2e} "
            f"(working precision {w['max_abs_beyond_rounding']:.2e}, measured {m['max_abs_beyond_rounding']:.2e}); "
            f"raw stated {stated[1]:.1e} applied {applied[1]:.2e}; "
            f"rel-L2 stated {stated[2]:.1e} applied {applied[2]:.2e} (measured {m['rel_l2']:.2e})")
    log(line)
    path = os.environ.get("FA2_GATE_LOG")
    if path:
        with open(path, "a") as f:
            f.write(line + "\n")


def check_bf16(name: str, got: np.ndarray, ref: np.ndarray, atol=ATOL_BF16, rl2=RL2_BF16,
               working: np.ndarray | None = None, cap_atol: float = CAP_ATOL,
               cap_rl2: float = CAP_RL2) -> dict:
    """Gate a bf16 result against the exact fp64 reference.

    ``working`` is the oracle's result at the method's working precision
    (bf16 P, O and dS at the method's rounding points).  When given, each gate
    is the stated tolerance or 1.5x the error that an exact execution at that
    precision makes, whichever is larger, capped at ``cap_atol`` (max-abs) and
    ``cap_rl2`` (relative L2); a widened gate is logged.
    """
    m = metrics(got, ref)
    stated = (atol, atol, rl2)
    raw_atol = atol
    if working is not None:
        w = metrics(round_bf16(working), ref)
        m["working_precision"] = w
        atol = min(cap_atol, max(atol, 1.5 * w["max_abs_beyond_rounding"]))
        raw_atol = min(cap_atol, max(raw_atol, 1.5 * w["max_abs"]))
        rl2 = min(cap_rl2, max(rl2, 1.5 * w["rel_l2"]))
        if (atol, raw_atol, rl2) != stated:
            _log_gate(name, m, stated, (atol, raw_atol, rl2))
    m["gate"] = {"beyond_rounding": atol, "raw": raw_atol, "rel_l2": rl2}
    assert m["finite"], f"{name}: non-finite output (unwritten or overflow)"
    assert m["max_abs_beyond_rounding"] <= atol, f"{name}: {m}"
    assert m["rel_l2"] <= rl2, f"{name}: {m}"
    if m["ref_max"] < 2.0:
        assert m["max_abs"] <= raw_atol, f"{name}: {m}"
    return m


def check_lse(name: str, got: np.ndarray, ref: np.ndarray, atol=ATOL_L) -> dict:
    got = np.asarray(got, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{name}: non-finite L"
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    assert err <= atol, f"{name}: max abs err {err:.3e}"
    return {"max_abs": err}


# ----------------------------------------------------------------------------- marshalling
def to_device_bf16(bits: np.ndarray, device="cuda"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(device)


def bf16_to_f64(t) -> np.ndarray:
    import torch
    assert t.dtype == torch.bfloat16
    bits = t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return inputs.bf16_bits_to_f64(bits)


def f32_to_f64(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)
