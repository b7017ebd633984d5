"""Acceptance gates comparing GPU output bits with the oracle (numpy only).

Contract gate (fp16 output): |C_gpu - C_ref| <= 1e-2 + 2e-3 |C_ref| per
element, and no negative (with ReLU) or NaN output.  Supplementary gates,
computed from the oracle's binary64 sums:
  G1  ||C_gpu - C_ref||_2 / ||C_ref||_2 <= 1e-3
  G2  |C_gpu - C_ref| <= ulp(C_ref) + 2 K 2^-24 (sum_k |A_ik B_kj| + |bias_j|)
      (the fp32 recursive-summation bound plus one output rounding each side)

bf16 output has 8 significand bits instead of 11: one output rounding is up
to 2^-7 relative instead of 2^-10, so its contract rtol and G1 bound are
2^-7 (one bf16 ulp relative to the bottom of a binade) instead of 2e-3 and
1e-3; the absolute tolerance and G2 keep their form.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

ATOL = 1e-2
RTOL = {"f16": 2e-3, "bf16": 2.0 ** -7}
G1_TOL = {"f16": 1e-3, "bf16": 2.0 ** -7}


def f16_values(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def bf16_values(bits: np.ndarray) -> np.ndarray:
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def ulpbf16(v: np.ndarray) -> np.ndarray:
    """Spacing of bf16 at |v| (2^-133 in the subnormal range)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    with np.errstate(divide="ignore", invalid="ignore"):
        _, e = np.frexp(a)                       # a in [2^(e-1), 2^e)
    sp = np.ldexp(1.0, np.maximum(e - 8, -133))
    return np.where(np.isfinite(a), sp, np.inf)


def ulp16(v: np.ndarray) -> np.ndarray:
    """Spacing of fp16 at |v| (2^-24 in the subnormal range)."""
    h = np.abs(v).astype(np.float16)
    with np.errstate(over="ignore", invalid="ignore"):
        sp = np.spacing(h).astype(np.float64)
    return np.where(np.isfinite(sp), sp, np.inf)


@dataclass
class GateReport:
    n: int
    max_abs_err: float
    contract_fail: int
    negative: int
    nan: int
    g1: float
    g2_fail: int
    bit_exact_frac: float
    g1_tol: float = G1_TOL["f16"]

    @property
    def ok(self) -> bool:
        return (self.contract_fail == 0 and self.negative == 0 and self.nan == 0
                and self.g1 <= self.g1_tol and self.g2_fail == 0)

    def __str__(self) -> str:
        return (f"n={self.n} max|err|={self.max_abs_err:.3g} contract_fail={self.contract_fail} "
                f"neg={self.negative} nan={self.nan} G1={self.g1:.3g} G2_fail={self.g2_fail} "
                f"bit_exact={self.bit_exact_frac:.4f}")


def gate(got_bits: np.ndarray, ref_bits: np.ndarray, K: int, abs_sum: np.ndarray | None = None,
         dtype: str = "f16", relu: bool = True) -> GateReport:
    """Gates for output bits of element type ``dtype`` ("f16" or "bf16");
    with ``relu`` every output must be non-negative (+0 included, -0 not)."""
    got_bits = np.asarray(got_bits, dtype=np.uint16).reshape(-1)
    ref_bits = np.asarray(ref_bits, dtype=np.uint16).reshape(-1)
    values = bf16_values if dtype == "bf16" else f16_values
    g = values(got_bits)
    r = values(ref_bits)
    nan = int(np.isnan(g).sum())
    # with ReLU a -0.0 counts too: the store must give +0
    negative = int(((got_bits & 0x8000) != 0).sum()) if relu else 0
    with np.errstate(invalid="ignore"):
        err = np.abs(g - r)
    err = np.where(np.isnan(err), np.inf, err)
    contract_fail = int((err > ATOL + RTOL[dtype] * np.abs(r)).sum())
    den = float(np.sqrt(np.sum(r * r)))
    num = float(np.sqrt(np.sum(np.where(np.isfinite(err), err, 1e30) ** 2)))
    g1 = num / den if den > 0 else (0.0 if num == 0 else np.inf)
    g2_fail = 0
    if abs_sum is not None:
        ulp = ulpbf16(r) if dtype == "bf16" else ulp16(r)
        bound = ulp + 2.0 * K * 2.0 ** -24 * np.asarray(abs_sum, dtype=np.float64).reshape(-1)
        g2_fail = int((err > bound).sum())
    return GateReport(n=got_bits.size, max_abs_err=float(err.max()) if err.size else 0.0,
                      contract_fail=contract_fail, negative=negative, nan=nan, g1=g1,
                      g2_fail=g2_fail,
                      bit_exact_frac=float(np.mean(got_bits == ref_bits)) if err.size else 1.0,
                      g1_tol=G1_TOL[dtype])
