"""Acceptance comparator (test infrastructure only).

The pass criterion is zero mismatching elements, not a mismatch fraction (ATOM
PR "test: add block-level DeepSeek-V4 attention test", section "Pass
criterion": a fraction-based idiom let a x1.05-perturbed tensor pass).

O passes when every element satisfies |O - ref| <= atol + rtol*|ref|
(atol = rtol = 1e-2); a NaN or Inf in O is a mismatch.  LSE passes when every
row satisfies |LSE - ref| <= 1e-3 (matching infinities pass).
"""
import dataclasses

import numpy as np

O_ATOL = 1e-2
O_RTOL = 1e-2
LSE_ATOL = 1e-3


@dataclasses.dataclass
class AcceptReport:
    ok: bool
    o_mismatch: int
    o_total: int
    lse_mismatch: int
    lse_total: int
    o_max_abs: float
    lse_max_abs: float

    def __str__(self):
        return (f"{'PASS' if self.ok else 'FAIL'}: O mismatch {self.o_mismatch}/{self.o_total} "
                f"(max abs {self.o_max_abs:.3g}), LSE mismatch {self.lse_mismatch}/{self.lse_total} "
                f"(max abs {self.lse_max_abs:.3g})")


def accept(o, lse, o_ref, lse_ref, atol=O_ATOL, rtol=O_RTOL, lse_atol=LSE_ATOL) -> AcceptReport:
    o = np.asarray(o, dtype=np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    lse_ref = np.asarray(lse_ref, dtype=np.float64)
    if o.shape != o_ref.shape or lse.shape != lse_ref.shape:
        raise ValueError(f"shape mismatch {o.shape}/{o_ref.shape}, {lse.shape}/{lse_ref.shape}")
    err = np.abs(o - o_ref)
    bad_o = ~(err <= atol + rtol * np.abs(o_ref))          # NaN compares False -> bad
    both_inf = np.isinf(lse) & np.isinf(lse_ref) & (np.sign(lse) == np.sign(lse_ref))
    with np.errstate(invalid="ignore"):
        lerr = np.where(both_inf, 0.0, np.abs(lse - lse_ref))
    bad_l = ~(lerr <= lse_atol)
    fin = np.isfinite(err)
    lfin = np.isfinite(lerr)
    return AcceptReport(
        ok=not bad_o.any() and not bad_l.any(),
        o_mismatch=int(bad_o.sum()), o_total=int(o.size),
        lse_mismatch=int(bad_l.sum()), lse_total=int(lse.size),
        o_max_abs=float(err[fin].max()) if fin.any() else float("nan"),
        lse_max_abs=float(lerr[lfin].max()) if lfin.any() else float("nan"))
