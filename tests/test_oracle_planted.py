"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case copies ``oracle/oracle.c``, plants one plausible mistake by a
textual replacement (a dropped term, a wrong sign, an off-by-one mask, a
wrong index or a transposed operand), compiles the copy, and checks that at
least one pin fails on it.  The real oracle is never modified.
"""
import os
import subprocess

import pytest

from oracle import oracle as orc
from tests import oracle_pins as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "oracle.c")

MUTATIONS = [
    ("scale dropped from the scores", "return scale * acc;", "return acc;"),
    ("causal mask off by one", "if (mk->causal && j > i) return 1;",
     "if (mk->causal && j > i + 1) return 1;"),
    ("block mask ignored", "if (mk->bm && !mk->bm[", "if (0 && mk->bm && !mk->bm["),
    ("block mask transposed",
     "mk->bm[(size_t)(i / ORACLE_SPARSE_BLOCK) * mk->nb + j / ORACLE_SPARSE_BLOCK]",
     "mk->bm[(size_t)(j / ORACLE_SPARSE_BLOCK) * mk->nb + i / ORACLE_SPARSE_BLOCK]"),
    ("masked row: exp(s - L) taken at s = L = -inf", "return s == -INFINITY ? 0.0 : exp(s - L);",
     "return exp(s - L);"),
    ("masked row: L = 0 instead of -inf", "if (m == -INFINITY) return -INFINITY;\n    double sum",
     "if (m == -INFINITY) return 0.0;\n    double sum"),
    ("masked row of the working-precision forward divided by l = 0",
     "if (m == -INFINITY) return -INFINITY;    /* every score masked: O_i = 0 */", ""),
    ("log2 instead of natural log in L", "return m + log(sum);", "return m + log2(sum);"),
    ("row maximum not subtracted inside the sum", "sum += exp(s[j] - m);", "sum += exp(s[j]);"),
    ("wrong GQA head mapping in the forward",
     "const double *Kh = head_ptr(K, b, hq / G, Hkv, N, d);\n            const double *Vh = head_ptr(V, b, hq / G, Hkv, N, d);\n            double *o = O",
     "const double *Kh = head_ptr(K, b, hq % Hkv, Hkv, N, d);\n            const double *Vh = head_ptr(V, b, hq / G, Hkv, N, d);\n            double *o = O"),
    ("value row index i instead of j", "const double *v = Vh + (size_t)j * d;\n        for (int t = 0; t < d; ++t) o[t] += p * v[t];",
     "const double *v = Vh + (size_t)i * d;\n        for (int t = 0; t < d; ++t) o[t] += p * v[t];"),
    ("D dropped from dS in dQ", "double ds = p * (dp - Dst[r]);", "double ds = p * dp;"),
    ("wrong sign of dS in dK", "double ds = p * (dp - Dst[(long)g * N + i]);",
     "double ds = p * (Dst[(long)g * N + i] - dp);"),
    ("D without the P weight", "D += p * dp;", "D += dp;"),
    ("dQ built from Q instead of K",
     "double ds = p * (dp - Dst[r]);\n                const double *k = Kh + (size_t)j * d;\n                for (int t = 0; t < d; ++t) dq[t] += ds * k[t];",
     "double ds = p * (dp - Dst[r]);\n                const double *k = Kh + (size_t)j * d;\n                for (int t = 0; t < d; ++t) dq[t] += ds * q[t];"),
    ("scale missing from dK", "for (int t = 0; t < d; ++t) dk[t] *= scale;\n    }\n}\n\n/*\n * Backward of one",
     "\n    }\n}\n\n/*\n * Backward of one"),
    ("dV uses the key-side row of dO (transposed operand)", "dv[t] += p * dOr[t];",
     "dv[t] += p * dOh[(size_t)j * d + t];"),
    ("dK sums over one query head of the group only",
     "for (int g = 0; g < G; ++g) {\n            int hq = hk * G + g;\n            const double *Qh = head_ptr(Q, b, hq, Hq, N, d);\n            const double *dOh = head_ptr(dO, b, hq, Hq, N, d);\n            for (int i = 0; i < N; ++i) {\n                const double *q = Qh + (size_t)i * d;\n                double sij",
     "for (int g = 0; g < 1; ++g) {\n            int hq = hk * G + g;\n            const double *Qh = head_ptr(Q, b, hq, Hq, N, d);\n            const double *dOh = head_ptr(dO, b, hq, Hq, N, d);\n            for (int i = 0; i < N; ++i) {\n                const double *q = Qh + (size_t)i * d;\n                double sij"),
    ("bf16 rounding to 7 significant bits", "u = (u + 0x7fffu + ((u >> 16) & 1u)) & 0xffff0000u;",
     "u = (u + 0xffffu + ((u >> 17) & 1u)) & 0xfffe0000u;"),
    ("bf16 rounding dropped from P of the working-precision forward", "double pb = round_bf16(p);\n        const double *v",
     "double pb = p;\n        const double *v"),
    ("bf16 rounding dropped from P of the working-precision dV", "double pb = round_bf16(p);\n                double ds",
     "double pb = p;\n                double ds"),
    ("working-precision D from the unrounded O", "D += dOr[t] * round_bf16(o[t]);", "D += dOr[t] * o[t];"),
    ("working-precision dS rounding dropped before dQ", "double ds = round_bf16(p * (dp - Dst[r]));",
     "double ds = p * (dp - Dst[r]);"),
    ("working-precision dS rounding dropped before dK",
     "double ds = round_bf16(p * (dp - Dst[(long)g * N + i]));", "double ds = p * (dp - Dst[(long)g * N + i]);"),
    ("backward from given outputs: the given O ignored in D", "for (int t = 0; t < d; ++t) D += g[t] * o[t];",
     "for (int t = 0; t < d; ++t) D += 0.0 * o[t];"),
    ("backward from given outputs: L of the wrong head group", "const double *Lg = L + row0;",
     "const double *Lg = L + (size_t)b * Hq * N;"),
    ("backward from given outputs: working precision ignored", "if (working_precision)\n",
     "if (0)\n"),
]


def _pins_fail(lib):
    failures = []
    for pin in pins.ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError) as e:
            failures.append(f"{pin.__name__}: {str(e)[:80]}")
    return failures


@pytest.mark.parametrize("desc,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(desc, old, new, tmp_path):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique/found: {old!r}"
    mutated = tmp_path / "oracle_mutant.c"
    mutated.write_text(src.replace(old, new))
    so = str(tmp_path / "liboracle_mutant.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-w",
                    "-o", so, str(mutated), "-lm"], check=True)
    lib = orc.load(so)
    failures = _pins_fail(lib)
    assert failures, f"planted mistake '{desc}' passed every pin"
