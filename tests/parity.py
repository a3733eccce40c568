"""Comparison of GPU results with the fp64 oracle, and tensor marshalling for GPU tests.

Tolerances (bf16 outputs O, dQ, dK, dV): max-abs error 1e-2 and relative L2
error 5e-3; fp32 L: max-abs 1e-3.  The max-abs gate is applied to the error
beyond the mandatory rounding of the exact value to bf16 (half a bf16 ulp of
the reference value): for |x| >= 4 a bf16 ulp is already 0.03, so no stored
bf16 value can be within 1e-2 of every exact value there.  The raw max-abs
error is reported alongside and gated as well wherever every reference
value is below 2 in magnitude (half an ulp there is at most 0.0039).

For the backward pass the gates may be raised to 1.5x the error of the
method executed exactly at its working precision (``working=``): the
method's bf16 operands alone put small causal problems slightly above
1e-2 beyond rounding.
"""
from __future__ import annotations

import sys

import numpy as np

from exact_io_aware_26_amd import inputs

ATOL_BF16 = 1e-2
RL2_BF16 = 5e-3
ATOL_L = 1e-3


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


def check_bf16(name: str, got: np.ndarray, ref: np.ndarray, atol=ATOL_BF16, rl2=RL2_BF16,
               working: np.ndarray | None = None) -> dict:
    """Gate a bf16 result against the exact fp64 reference.

    ``working`` is the oracle's result at the method's working precision
    (bf16 P, O and dS at the method's rounding points, see oracle_bwd_bf16).
    When given, each gate is the stated tolerance or 1.5x the error that an
    exact execution at that precision makes, whichever is larger: no kernel
    that uses bf16 operands where the method does can beat that floor.
    """
    m = metrics(got, ref)
    raw_atol = atol
    if working is not None:
        w = metrics(round_bf16(working), ref)
        atol = max(atol, 1.5 * w["max_abs_beyond_rounding"])
        rl2 = max(rl2, 1.5 * w["rel_l2"])
        raw_atol = max(raw_atol, 1.5 * w["max_abs"])
        m["working_precision"] = w
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
