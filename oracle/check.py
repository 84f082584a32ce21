"""Result checker for the SGEMM oracle (TEST INFRASTRUCTURE ONLY).

Gate for C = A B, per element:

    |C_gpu - C_ref| <= 4 * K * 2**-24 * S,   S = sum_k |a_ik b_kj|.

This is the componentwise forward error bound of a length-K float dot product
(|fl(x.y) - x.y| <= gamma_K * sum |x_i y_i| with gamma_K = K u / (1 - K u),
u = 2**-24; Higham, "Accuracy and Stability of Numerical Algorithms", 2nd ed.,
section 3.1), which holds for every summation order; the factor 4 leaves room
for the matrix unit's internal ordering and for the reference's own (far
smaller) double-precision rounding.  With K = 0 the bound is 0 and C must be
exactly 0.

Gate for the general form C = alpha op(A) op(B) + beta C0, per element:

    |C_gpu - C_ref| <= 4 * K * 2**-24 * S + 2 * 2**-24 * E,

with S = |alpha| sum_k |a_ik b_kj| (the accumulation, as above) and
E = |alpha sum_k a_ik b_kj| + |beta C0_ij| (the final scaling and the final
addition, each rounded once to float: one unit roundoff of the value rounded
each time; the factor 2 is the same kind of slack).  With K = 0 or
alpha = 0 only the E term remains.

Non-finite values: any NaN or infinity in C_gpu is a violation, even where the
reference is not finite too.  These gates are for finite inputs; NaN and
infinity propagation is compared separately, as a pattern (the tests of
special values).

Also reported, for information, is the relative-error figure of amittech.dev,
"3.5 Project: tiled matrix multiplication", section "starter scaffolding"
(the tolerance checker): max |g - r| / max(|r|, 1e-6).  That figure is not a
gate here, because on zero-mean inputs some outputs sit near zero and a
correct float result can exceed a fixed relative tolerance there.
"""
from __future__ import annotations

import numpy as np

U = 2.0 ** -24
SLACK = 4.0
SLACK_E = 2.0


def bound(S: np.ndarray, K: int) -> np.ndarray:
    """Allowed absolute error per element for inner dimension K."""
    return SLACK * K * U * np.asarray(S, dtype=np.float64)


def bound_ex(S: np.ndarray, E: np.ndarray, K: int) -> np.ndarray:
    """Allowed absolute error per element of the general form."""
    return bound(S, K) + SLACK_E * U * np.asarray(E, dtype=np.float64)


def _report(C_gpu, C_ref, b) -> dict:
    g = np.asarray(C_gpu, dtype=np.float64)
    r = np.asarray(C_ref, dtype=np.float64)
    if g.shape != r.shape:
        raise ValueError(f"shape mismatch {g.shape} vs {r.shape}")
    b = np.broadcast_to(np.asarray(b, dtype=np.float64), g.shape)
    err = np.abs(g - r)
    bad = ~np.isfinite(g)
    viol = bad | (err > b)
    with np.errstate(divide="ignore", invalid="ignore"):
        util = np.where(b > 0, err / np.where(b > 0, b, 1.0), np.where(err == 0, 0.0, np.inf))
        rel = err / np.maximum(np.abs(r), 1e-6)
    fin = ~bad
    return {
        "ok": bool(not viol.any()),
        "n": int(g.size),
        "n_violations": int(viol.sum()),
        "n_nonfinite": int(bad.sum()),
        "max_bound_util": float(util[fin].max()) if fin.any() else 0.0,
        "max_abs_err": float(err[fin].max()) if fin.any() else 0.0,
        "max_rel_err_page": float(rel[fin].max()) if fin.any() else 0.0,
    }


def check(C_gpu, C_ref, S, K: int) -> dict:
    """Compare a float result of C = A B with the double reference; returns a
    report whose ``ok`` is True when every element is finite and within
    4 K 2^-24 S."""
    return _report(C_gpu, C_ref, bound(S, K))


def check_ex(C_gpu, C_ref, S, E, K: int) -> dict:
    """Gate for C = alpha op(A) op(B) + beta C0: every element finite and
    within 4 K 2^-24 S + 2 * 2^-24 E (S and E as the oracle's general form
    returns them)."""
    return _report(C_gpu, C_ref, bound_ex(S, E, K))
