"""Result checker for the SGEMM oracle (TEST INFRASTRUCTURE ONLY).

Gate, per element:  |C_gpu - C_ref| <= 4 * K * 2**-24 * S,  S = sum_k |a_ik b_kj|.

This is the componentwise forward error bound of a length-K float dot product
(|fl(x.y) - x.y| <= gamma_K * sum |x_i y_i| with gamma_K = K u / (1 - K u),
u = 2**-24; Higham, "Accuracy and Stability of Numerical Algorithms", 2nd ed.,
section 3.1), which holds for every summation order; the factor 4 leaves room
for the matrix unit's internal ordering and for the reference's own (far
smaller) double-precision rounding.  With K = 0 the bound is 0 and C must be
exactly 0.

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


def bound(S: np.ndarray, K: int) -> np.ndarray:
    """Allowed absolute error per element for inner dimension K."""
    return SLACK * K * U * np.asarray(S, dtype=np.float64)


def check(C_gpu, C_ref, S, K: int) -> dict:
    """Compare a float result with the double reference; returns a report.

    ``ok`` is True when every element is finite and within the bound."""
    g = np.asarray(C_gpu, dtype=np.float64)
    r = np.asarray(C_ref, dtype=np.float64)
    if g.shape != r.shape:
        raise ValueError(f"shape mismatch {g.shape} vs {r.shape}")
    b = bound(S, K)
    err = np.abs(g - r)
    nan = ~np.isfinite(g)
    viol = nan | (err > b)
    with np.errstate(divide="ignore", invalid="ignore"):
        util = np.where(b > 0, err / np.where(b > 0, b, 1.0), np.where(err == 0, 0.0, np.inf))
        rel = err / np.maximum(np.abs(r), 1e-6)
    finite_util = util[~nan]
    return {
        "ok": bool(not viol.any()),
        "n": int(g.size),
        "n_violations": int(viol.sum()),
        "n_nonfinite": int(nan.sum()),
        "max_bound_util": float(finite_util.max()) if finite_util.size else 0.0,
        "max_abs_err": float(err[~nan].max()) if (~nan).any() else 0.0,
        "max_rel_err_page": float(rel[~nan].max()) if (~nan).any() else 0.0,
    }


def check_ex(C_gpu, C_ref, S, E, K: int) -> dict:
    """Gate for C = alpha op(A) op(B) + beta C0:
    |C - C_ref| <= 4 K 2^-24 S + 2 * 2^-24 E, where S = |alpha| sum|ab| covers
    the dot product's accumulation and E = |alpha sum ab| + |beta C0| the
    final scaling and addition (one rounding each)."""
    g = np.asarray(C_gpu, dtype=np.float64)
    r = np.asarray(C_ref, dtype=np.float64)
    b = SLACK * K * U * np.asarray(S, dtype=np.float64) + 2 * U * np.asarray(E, dtype=np.float64)
    err = np.abs(g - r)
    nan = ~np.isfinite(g)
    viol = nan | (err > b)
    with np.errstate(divide="ignore", invalid="ignore"):
        util = np.where(b > 0, err / np.where(b > 0, b, 1.0), np.where(err == 0, 0.0, np.inf))
    fu = util[~nan]
    return {"ok": bool(not viol.any()), "n": int(g.size), "n_violations": int(viol.sum()),
            "n_nonfinite": int(nan.sum()), "max_bound_util": float(fu.max()) if fu.size else 0.0}
