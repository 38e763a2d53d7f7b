"""Code-by-code check of GPTQ codes against the oracle (no GPU needed).

GPTQ rounds the rows of each output channel in order, and every rounding
error moves the later rows ("06 -- SmoothQuant", section 10; the published
GPTQ algorithm).  Two evaluations that sum the Hessian, the factorizations and
the updates in different orders agree to about 1e-13 relative, so they take
the same codes except where a quotient lies on a rounding boundary; there they
may legitimately part, and from then on that channel follows a different (and
equally valid) trajectory.

check_gptq_codes therefore checks every code: at each column's first
difference, the oracle's quotient must be within 1e-7 of a half-integer; the
oracle then re-runs that column with the other side's codes up to and
including that row, and the check continues from there, until the column
agrees to its end.  No code goes unchecked after a legitimate parting.
"""
from __future__ import annotations

import numpy as np

import oracle

TIE_BAND = 1e-7


def _near_tie(v: float) -> bool:
    return abs(abs(v - np.floor(v)) - 0.5) < TIE_BAND


def check_gptq_codes(q_gpu, w_cols, U, dead, *, max_partings: int = 16) -> int:
    """q_gpu [n, K] int8: the codes to check for the output channels whose
    migrated weight is w_cols [K, n] fp32; (U, dead) from oracle.gptq_factor.
    Raises AssertionError at the first code the oracle cannot account for.
    Returns the number of partings at near-ties over all columns."""
    q_gpu = np.asarray(q_gpu, np.int8)
    W = np.asarray(w_cols, np.float32)
    K, n = W.shape
    assert q_gpu.shape == (n, K)
    q_ref, _, quot = oracle.gptq_round(W, U, dead, return_quotients=True)
    partings = 0
    for c in np.nonzero((q_gpu != q_ref).any(axis=1))[0]:
        col = W[:, [c]]
        ref_c, quot_c = q_ref[c], quot[:, c]
        upto = 0
        for _ in range(max_partings + 1):
            diff = np.nonzero(q_gpu[c] != ref_c)[0]
            if diff.size == 0:
                break
            j = int(diff[0])
            assert j >= upto
            assert _near_tie(float(quot_c[j])), (
                f"channel {int(c)} row {j}: code {int(q_gpu[c, j])} vs oracle "
                f"{int(ref_c[j])}, quotient {float(quot_c[j])!r} is not at a rounding boundary")
            partings += 1
            upto = j + 1
            r, _, qt = oracle.gptq_round(col, U, dead, return_quotients=True,
                                         force_codes=q_gpu[[c]], force_rows=np.array([upto]))
            ref_c, quot_c = r[0], qt[:, 0]
        else:
            raise AssertionError(f"channel {int(c)} parted more than {max_partings} times")
    return partings
