"""Pins that tie the result checker (oracle/check.py) to facts fixed outside
its own code.

Each ``pin_*`` takes a checker module (so the mutation test can run the same
pins against deliberately broken copies of it) and raises AssertionError when
the checker disagrees with:

* hand-worked bounds: small cases whose S, E and allowed error are worked out
  by hand in the comments (u = 2**-24), with a result exactly at the bound
  (accepted), one unit of 2**-24 past it (rejected) and the same distance on
  the other side (rejected);
* the degenerate forms: K = 0 and alpha = 0 leave only the final rounding,
  2 u |beta C0|; the plain product at K = 0 must be exactly zero;
* a case where E dominates S, so that a checker with S and E exchanged
  accepts an error the true bound rejects;
* non-finite results (NaN, +-infinity) are always violations;
* float arithmetic itself: a float32 computation (products and sums rounded
  to float in ascending k, then alpha and beta applied as a fused
  multiply-add) lies within the bound of the exact rational result, in every
  case tried, whichever order it sums in.

Numbers below are exact in double, so "exactly at the bound" is exact.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

u = 2.0 ** -24


def _ok(rep):
    return bool(rep["ok"])


def pin_plain_hand_bound(chk):
    # A = [1, 1], B = [1, 1]^T: K = 2, sum = 2, S = 2.
    # Allowed error 4 * K * u * S = 4 * 2 * 2 * u = 16 u.
    r, S, K = np.array([2.0]), np.array([2.0]), 2
    assert _ok(chk.check(np.array([2.0 + 16 * u]), r, S, K)), "error at the bound rejected"
    assert not _ok(chk.check(np.array([2.0 + 17 * u]), r, S, K)), "error past the bound accepted"
    assert not _ok(chk.check(np.array([2.0 - 17 * u]), r, S, K)), "negative error past the bound accepted"
    # A row of K = 1000 terms a_k b_k = +-0.5 summing to 0: S = 500, bound
    # 4 * 1000 * 500 u = 2e6 u, about 0.119.
    r0, S0 = np.array([0.0]), np.array([500.0])
    assert _ok(chk.check(np.array([2e6 * u]), r0, S0, 1000))
    assert not _ok(chk.check(np.array([-2.0000001e6 * u]), r0, S0, 1000))


def pin_plain_k_zero(chk):
    # K = 0: the empty sum is exactly 0, S = 0, nothing may differ.
    z = np.zeros((2, 2))
    assert _ok(chk.check(np.zeros((2, 2), np.float32), z, z, 0))
    assert not _ok(chk.check(np.full((2, 2), 1e-30, np.float32), z, z, 0))


def pin_nonfinite_rejected(chk):
    r, S = np.array([1.0, 2.0, 3.0]), np.array([10.0, 10.0, 10.0])
    for bad in (np.nan, np.inf, -np.inf):
        g = np.array([1.0, bad, 3.0])
        rep = chk.check(g, r, S, 4)
        assert not _ok(rep) and rep["n_nonfinite"] == 1, f"{bad} accepted by check"
        rep = chk.check_ex(g, r, S, np.abs(r), 4)
        assert not _ok(rep) and rep["n_nonfinite"] == 1, f"{bad} accepted by check_ex"


def pin_ex_hand_bound(chk):
    # A = [1, 1], B = [1, 1]^T, alpha = 1, beta = 1, C0 = 1: K = 2,
    # sum = 2, C = 3, S = |alpha| * 2 = 2, E = |alpha * 2| + |beta * 1| = 3.
    # Allowed error 4 * 2 * u * 2 + 2 * u * 3 = 16 u + 6 u = 22 u.
    r, S, E, K = np.array([3.0]), np.array([2.0]), np.array([3.0]), 2
    assert _ok(chk.check_ex(np.array([3.0 + 22 * u]), r, S, E, K)), "error at the bound rejected"
    assert not _ok(chk.check_ex(np.array([3.0 + 23 * u]), r, S, E, K)), "error past the bound accepted"
    assert not _ok(chk.check_ex(np.array([3.0 - 23 * u]), r, S, E, K)), "negative error past the bound accepted"


def pin_ex_k_zero_and_alpha_zero(chk):
    # K = 0, beta = 0.5, C0 = 3: C = 1.5, S = 0, E = 1.5; allowed 2 u * 1.5 = 3 u.
    r, S, E = np.array([1.5]), np.array([0.0]), np.array([1.5])
    assert _ok(chk.check_ex(np.array([1.5 + 3 * u]), r, S, E, 0))
    assert not _ok(chk.check_ex(np.array([1.5 + 4 * u]), r, S, E, 0))
    # alpha = 0, K = 5, beta = 2, C0 = 1: S = |alpha| sum|ab| = 0, E = 2;
    # allowed 2 u * 2 = 4 u, whatever K is.
    r, S, E = np.array([2.0]), np.array([0.0]), np.array([2.0])
    assert _ok(chk.check_ex(np.array([2.0 + 4 * u]), r, S, E, 5))
    assert not _ok(chk.check_ex(np.array([2.0 + 5 * u]), r, S, E, 5))


def pin_ex_e_dominates(chk):
    # A = [2^-20, 0], B = [1, 1]^T, alpha = 1, beta = 1, C0 = 1000 - 2^-20:
    # K = 2, sum = 2^-20 = S, C = 1000, E = 2^-20 + (1000 - 2^-20) = 1000.
    # Allowed 4 * 2 * u * 2^-20 + 2 * u * 1000 = 2000 u + 8 * 2^-44.  With S
    # and E exchanged it would be 8000 u: an error of 3000 u tells them apart.
    S = np.array([2.0 ** -20])
    E = np.array([1000.0])
    r = np.array([1000.0])
    assert _ok(chk.check_ex(np.array([1000.0 + 2000 * u]), r, S, E, 2))
    assert not _ok(chk.check_ex(np.array([1000.0 + 3000 * u]), r, S, E, 2))
    # The reverse: S large, E small.  A = [1, -1], B = [1, 1]^T, alpha = 1,
    # beta = 1, C0 = 1: sum = 0, C = 1, S = 2, E = 0 + 1 = 1.  Allowed
    # 4 * 2 * u * 2 + 2 * u * 1 = 18 u; exchanged, 4 * 2 * u * 1 + 2 * u * 2 = 12 u.
    r, S, E = np.array([1.0]), np.array([2.0]), np.array([1.0])
    assert _ok(chk.check_ex(np.array([1.0 + 18 * u]), r, S, E, 2))
    assert not _ok(chk.check_ex(np.array([1.0 + 19 * u]), r, S, E, 2))


def _exact(A, B, alpha, beta, C0):
    """Exact rational alpha A B + beta C0 with S and E, element by element."""
    M, K = A.shape
    N = B.shape[1]
    a = Fraction(float(alpha))
    b = Fraction(float(beta))
    C = np.empty((M, N))
    S = np.empty((M, N))
    E = np.empty((M, N))
    for i in range(M):
        for j in range(N):
            terms = [Fraction(float(A[i, k])) * Fraction(float(B[k, j])) for k in range(K)]
            s = sum(terms, Fraction(0))
            c0 = b * Fraction(float(C0[i, j]))
            C[i, j] = float(a * s + c0)
            S[i, j] = float(abs(a) * sum((abs(t) for t in terms), Fraction(0)))
            E[i, j] = float(abs(a * s) + abs(c0))
    return C, S, E


def _float32_gemm(A, B, alpha, beta, C0, order):
    """C = alpha A B + beta C0 computed in float32: each product and each
    partial sum rounded to float, k in the given order; then alpha * sum
    rounded, then beta * C0 added with one rounding (a fused multiply-add)."""
    acc = np.zeros((A.shape[0], B.shape[1]), dtype=np.float32)
    for k in order:
        acc = (acc + np.outer(A[:, k], B[k, :]).astype(np.float32)).astype(np.float32)
    v = (np.float32(alpha) * acc).astype(np.float32)
    return (np.float64(beta) * C0.astype(np.float64) + v.astype(np.float64)).astype(np.float32)


def pin_float32_results_accepted(chk):
    rng = np.random.default_rng(12)
    for (M, N, K, alpha, beta) in [(3, 4, 300, 1.0, 0.0), (2, 3, 257, -1.5, 0.75), (3, 2, 64, 0.3, -2.0)]:
        A = (rng.random((M, K), dtype=np.float32) * 2 - 1).astype(np.float32)
        B = (rng.random((K, N), dtype=np.float32) * 2 - 1).astype(np.float32)
        C0 = (rng.standard_normal((M, N)) * 4).astype(np.float32)
        ref, S, E = _exact(A, B, alpha, beta, C0)
        for order in (range(K), range(K - 1, -1, -1)):
            got = _float32_gemm(A, B, alpha, beta, C0, order)
            rep = chk.check_ex(got, ref, S, E, K)
            assert _ok(rep) and rep["max_bound_util"] < 1.0, (M, N, K, rep)
            if beta == 0.0 and alpha == 1.0:
                rep = chk.check(got, ref, S, K)
                assert _ok(rep), (M, N, K, rep)


ALL_PINS = [pin_plain_hand_bound, pin_plain_k_zero, pin_nonfinite_rejected, pin_ex_hand_bound,
            pin_ex_k_zero_and_alpha_zero, pin_ex_e_dominates, pin_float32_results_accepted]
