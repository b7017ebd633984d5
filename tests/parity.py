"""Acceptance gates comparing GPU output bits with the oracle (numpy only).

Contract gate: |C_gpu - C_ref| <= 1e-2 + 2e-3 |C_ref| per element, and no
negative or NaN output.  Supplementary gates, computed from the oracle's
binary64 sums:
  G1  ||C_gpu - C_ref||_2 / ||C_ref||_2 <= 1e-3
  G2  |C_gpu - C_ref| <= ulp16(C_ref) + 2 K 2^-24 sum_k |A_ik B_kj|
      (the fp32 recursive-summation bound plus one fp16 rounding each side)
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

ATOL = 1e-2
RTOL = 2e-3
G1_TOL = 1e-3


def f16_values(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


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

    @property
    def ok(self) -> bool:
        return (self.contract_fail == 0 and self.negative == 0 and self.nan == 0
                and self.g1 <= G1_TOL and self.g2_fail == 0)

    def __str__(self) -> str:
        return (f"n={self.n} max|err|={self.max_abs_err:.3g} contract_fail={self.contract_fail} "
                f"neg={self.negative} nan={self.nan} G1={self.g1:.3g} G2_fail={self.g2_fail} "
                f"bit_exact={self.bit_exact_frac:.4f}")


def gate(got_bits: np.ndarray, ref_bits: np.ndarray, K: int, abs_sum: np.ndarray | None = None
         ) -> GateReport:
    got_bits = np.asarray(got_bits, dtype=np.uint16).reshape(-1)
    ref_bits = np.asarray(ref_bits, dtype=np.uint16).reshape(-1)
    g = f16_values(got_bits)
    r = f16_values(ref_bits)
    nan = int(np.isnan(g).sum())
    negative = int(((got_bits & 0x8000) != 0).sum())  # -0.0 counts: the store must give +0
    with np.errstate(invalid="ignore"):
        err = np.abs(g - r)
    err = np.where(np.isnan(err), np.inf, err)
    contract_fail = int((err > ATOL + RTOL * np.abs(r)).sum())
    den = float(np.sqrt(np.sum(r * r)))
    num = float(np.sqrt(np.sum(np.where(np.isfinite(err), err, 1e30) ** 2)))
    g1 = num / den if den > 0 else (0.0 if num == 0 else np.inf)
    g2_fail = 0
    if abs_sum is not None:
        bound = ulp16(r) + 2.0 * K * 2.0 ** -24 * np.asarray(abs_sum, dtype=np.float64).reshape(-1)
        g2_fail = int((err > bound).sum())
    return GateReport(n=got_bits.size, max_abs_err=float(err.max()) if err.size else 0.0,
                      contract_fail=contract_fail, negative=negative, nan=nan, g1=g1,
                      g2_fail=g2_fail,
                      bit_exact_frac=float(np.mean(got_bits == ref_bits)) if err.size else 1.0)
