"""Pins that tie the CPU oracle to facts fixed outside its own code.

Each ``pin_*`` function takes a loaded oracle library (so the mutation test
can run the same pins against deliberately broken builds of the oracle) and
raises AssertionError when the oracle disagrees with:

* hand-computed products (tests/golden/hand_products.txt);
* the exact rational product (Python ``fractions``), within the double
  rounding bound K * 2**-53 * sum|a b|, on every shape up to 4 x 4 x 4 and a
  few larger ragged ones, with NaN-filled leading-dimension padding;
* closed forms: A * I = A and I * B = B exactly; B = ones gives row sums of A;
* a library routine on a case that reduces to it: integer inputs make the
  product exact, equal to numpy's int64 matrix product;
* degenerate sizes: K = 0 gives zeros, M = 0 or N = 0 gives an empty result;
* for the compute-roof probes: closed forms of the multiply-add chain, each
  step rounded once from the exact rational value, and hand-worked cases of
  the 32 x 2 by 2 x 32 product.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np

import oracle
from roofline_sgemm_f32_amd.inputs import as_numpy, make_operands

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_hand_cases():
    cases = []
    with open(os.path.join(GOLDEN, "hand_products.txt")) as f:
        lines = [ln.split("#")[0].strip() for ln in f]
    lines = [ln for ln in lines if ln]
    i = 0
    while i < len(lines):
        head = lines[i].split()
        assert head[0] == "case", head
        name, M, N, K = head[1], int(head[2]), int(head[3]), int(head[4])
        i += 1
        rows = [[float(v) for v in lines[i + r].split()] for r in range(M + K + M)]
        i += M + K + M
        A = np.array(rows[:M], dtype=np.float32).reshape(M, K)
        B = np.array(rows[M:M + K], dtype=np.float32).reshape(K, N)
        C = np.array(rows[M + K:], dtype=np.float64).reshape(M, N)
        cases.append((name, A, B, C))
    return cases


def exact_product(A: np.ndarray, B: np.ndarray):
    """Exact rational A*B and sum|a b|, element by element."""
    M, K = A.shape
    N = B.shape[1]
    Af = [[Fraction(float(A[i, k])) for k in range(K)] for i in range(M)]
    Bf = [[Fraction(float(B[k, j])) for j in range(N)] for k in range(K)]
    C = [[sum((Af[i][k] * Bf[k][j] for k in range(K)), Fraction(0)) for j in range(N)]
         for i in range(M)]
    S = [[sum((abs(Af[i][k] * Bf[k][j]) for k in range(K)), Fraction(0)) for j in range(N)]
         for i in range(M)]
    return C, S


def _assert_close_exact(name, got, got_S, C, S, K):
    M = len(C)
    N = len(C[0]) if M else 0
    tol_scale = max(K, 1) * 2.0 ** -53
    for i in range(M):
        for j in range(N):
            tol = float(S[i][j]) * tol_scale
            assert abs(Fraction(float(got[i, j])) - C[i][j]) <= Fraction(tol), \
                f"{name}: C[{i},{j}]={got[i, j]!r} exact={float(C[i][j])!r}"
            if got_S is not None:
                assert abs(Fraction(float(got_S[i, j])) - S[i][j]) <= Fraction(tol), \
                    f"{name}: S[{i},{j}]={got_S[i, j]!r} exact={float(S[i][j])!r}"


def pin_hand_examples(lib):
    for name, A, B, C in load_hand_cases():
        got, S = oracle.sgemm_f64(A, B, lib=lib, threads=2)
        assert np.array_equal(got, C), f"{name}: {got} != {C}"
        rows, _ = oracle.sgemm_rows_f64(A, B, np.arange(A.shape[0]), lib=lib, threads=2)
        assert np.array_equal(rows, C), f"{name} (rows): {rows} != {C}"
        ii, jj = np.meshgrid(np.arange(A.shape[0]), np.arange(B.shape[1]), indexing="ij")
        ent, _ = oracle.sgemm_entries_f64(A, B, ii.ravel(), jj.ravel(), lib=lib)
        assert np.array_equal(ent.reshape(C.shape), C), f"{name} (entries)"


def _shapes_small():
    for M in range(1, 5):
        for N in range(1, 5):
            for K in range(1, 5):
                yield M, N, K
    yield from [(5, 7, 3), (3, 2, 9), (6, 5, 17), (2, 9, 33)]


def pin_bruteforce_exact(lib):
    for t, (M, N, K) in enumerate(_shapes_small()):
        # Leading dimensions with NaN padding catch any read past a row.
        A, B = make_operands(M, N, K, "uniform", seed=1000 + t, lda=K + (t % 3), ldb=N + (t % 2))
        A, B = as_numpy(A), as_numpy(B)
        C, S = exact_product(A, B)
        got, got_S = oracle.sgemm_f64(A, B, lib=lib, threads=3)
        _assert_close_exact(f"full {M}x{N}x{K}", got, got_S, C, S, K)
        rows = np.arange(M)[::-1].copy()
        gr, gs = oracle.sgemm_rows_f64(A, B, rows, lib=lib, threads=2)
        _assert_close_exact(f"rows {M}x{N}x{K}", gr, gs, [C[r] for r in rows],
                            [S[r] for r in rows], K)
        ii, jj = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
        ge, gse = oracle.sgemm_entries_f64(A, B, ii.ravel(), jj.ravel(), lib=lib)
        _assert_close_exact(f"entries {M}x{N}x{K}", ge.reshape(M, N), gse.reshape(M, N), C, S, K)


def pin_identity(lib):
    A, B = make_operands(19, 23, 11, "uniform", seed=7)
    A, B = as_numpy(A), as_numpy(B)
    I_k = np.eye(11, dtype=np.float32)
    got, _ = oracle.sgemm_f64(A, I_k, lib=lib)  # A * I = A
    assert np.array_equal(got, A.astype(np.float64)), "A*I != A"
    got, _ = oracle.sgemm_f64(I_k, B, lib=lib)  # I * B = B
    assert np.array_equal(got, B.astype(np.float64)), "I*B != B"


def pin_all_ones(lib):
    # B = ones: every entry of row i is the sum of row i of A.
    A, _ = make_operands(13, 1, 57, "uniform", seed=8)
    A = as_numpy(A)
    ones = np.ones((57, 9), dtype=np.float32)
    got, S = oracle.sgemm_f64(A, ones, lib=lib)
    for i in range(13):
        exact = math.fsum(float(v) for v in A[i])
        tol = 57 * 2.0 ** -53 * float(np.abs(A[i].astype(np.float64)).sum())
        assert np.all(np.abs(got[i] - exact) <= tol), f"row {i} sum"
    # A = ones: every entry of column j is the sum of column j of B.
    _, B = make_operands(1, 12, 40, "int", seed=9)
    B = as_numpy(B)
    got, _ = oracle.sgemm_f64(np.ones((5, 40), dtype=np.float32), B, lib=lib)
    colsum = B.astype(np.int64).sum(axis=0)
    assert np.array_equal(got, np.tile(colsum, (5, 1)).astype(np.float64)), "column sums"


def pin_integer_library(lib):
    # Integer inputs in [-2, 2]: the product is an exact small integer, so it
    # must equal numpy's exact int64 product bit for bit.
    for (M, N, K, lda, ldb) in [(37, 29, 41, 41, 29), (64, 65, 63, 70, 66), (1, 200, 300, 300, 201)]:
        A, B = make_operands(M, N, K, "int", seed=M * 7 + N, lda=lda, ldb=ldb)
        A, B = as_numpy(A), as_numpy(B)
        want = np.matmul(A.astype(np.int64), B.astype(np.int64))
        want_abs = np.matmul(np.abs(A.astype(np.int64)), np.abs(B.astype(np.int64)))
        got, S = oracle.sgemm_f64(A, B, lib=lib, threads=4)
        assert np.array_equal(got, want.astype(np.float64)), f"int {M}x{N}x{K}"
        assert np.array_equal(S, want_abs.astype(np.float64)), f"int bound {M}x{N}x{K}"


def pin_degenerate(lib):
    A = np.zeros((4, 0), dtype=np.float32)
    B = np.zeros((0, 6), dtype=np.float32)
    got, S = oracle.sgemm_f64(A, B, lib=lib)
    assert got.shape == (4, 6) and np.all(got == 0) and np.all(S == 0), "K=0 must give zeros"
    got, _ = oracle.sgemm_f64(np.zeros((0, 3), np.float32), np.ones((3, 5), np.float32), lib=lib)
    assert got.shape == (0, 5)
    got, _ = oracle.sgemm_f64(np.ones((2, 3), np.float32), np.zeros((3, 0), np.float32), lib=lib)
    assert got.shape == (2, 0)


ALL_PINS = [pin_hand_examples, pin_bruteforce_exact, pin_identity, pin_all_ones,
            pin_integer_library, pin_degenerate]


# --- the compute-roof probes' oracle ---------------------------------------

def round_to_f32(q: Fraction) -> np.float32:
    """Round an exact rational to the nearest float32 (ties to even)."""
    f = np.float32(float(q))
    lo, hi = (np.nextafter(f, np.float32(-np.inf)), f) if Fraction(float(f)) > q else \
             (f, np.nextafter(f, np.float32(np.inf)))
    dl, dh = q - Fraction(float(lo)), Fraction(float(hi)) - q
    if dl != dh:
        return lo if dl < dh else hi
    return lo if (int(lo.view(np.uint32)) & 1) == 0 else hi


def pin_fma_chain_exact_rounding(lib):
    # Each step is the exact value acc * x + y rounded once to float32.
    x, y = np.float32(0.999), np.float32(0.001)
    got = oracle.fma_chain_f32(300, float(x), float(y), 16, lib=lib)
    for j in range(16):
        acc = np.float32(0.0625) * np.float32(j + 1)
        for _ in range(300):
            acc = round_to_f32(Fraction(float(acc)) * Fraction(float(x)) + Fraction(float(y)))
        assert got[j] == acc, (j, got[j], acc)


def pin_fma_chain_closed_forms(lib):
    # x = 1, y = 1: each step adds 1 exactly (values stay below 2^24).
    got = oracle.fma_chain_f32(1000, 1.0, 1.0, 16, lib=lib)
    assert np.array_equal(got, np.float32(0.0625) * np.arange(1, 17, dtype=np.float32) + 1000), got
    # x = 2, y = 0: doubling is exact.
    got = oracle.fma_chain_f32(20, 2.0, 0.0, 16, lib=lib)
    assert np.array_equal(got, np.float32(0.0625) * np.arange(1, 17, dtype=np.float32) * 2 ** 20), got
    # x = 0.5, y = 0.5 from a = 1/16: a_n = 1 - (15/16) 2^-n, exact for small n.
    got = oracle.fma_chain_f32(5, 0.5, 0.5, 1, lib=lib)
    assert got[0] == np.float32(1 - 15 / 16 * 2 ** -5), got
    # zero iterations return the starting values.
    assert np.array_equal(oracle.fma_chain_f32(0, 3.0, 7.0, 4, lib=lib),
                          np.float32(0.0625) * np.arange(1, 5, dtype=np.float32))


def pin_mfma_probe_products(lib):
    # All ones: every entry is iters * 2 (two k terms).
    D = oracle.mfma_probe_f64(3, np.ones(64), np.ones(64), lib=lib)
    assert np.all(D == 6.0)
    # A[5][0] = 1 (a_vals[5]) and B[0][7] = 1 (b_vals[7]): only D[5][7] = iters.
    a = np.zeros(64); a[5] = 1
    b = np.zeros(64); b[7] = 1
    D = oracle.mfma_probe_f64(9, a, b, lib=lib)
    want = np.zeros((32, 32)); want[5, 7] = 9
    assert np.array_equal(D, want)
    # Mismatched k (A uses k = 0, B uses k = 1): zero.
    b = np.zeros(64); b[7 + 32] = 1
    assert np.all(oracle.mfma_probe_f64(9, a, b, lib=lib) == 0)
    # A[i][1] = a_vals[i + 32], B[1][j] = b_vals[j + 32]: an outer product.
    a = np.zeros(64); a[32:] = np.arange(32)
    b = np.zeros(64); b[32:] = np.arange(32) - 16
    D = oracle.mfma_probe_f64(2, a, b, lib=lib)
    assert np.array_equal(D, 2 * np.outer(np.arange(32), np.arange(32) - 16))


ALL_PINS += [pin_fma_chain_closed_forms, pin_fma_chain_exact_rounding, pin_mfma_probe_products]


# --- the general form C = alpha op(A) op(B) + beta C0 ----------------------

def _ex_cases():
    # (transa, transb, alpha, beta)
    for ta in (False, True):
        for tb in (False, True):
            for alpha, beta in ((1.0, 0.0), (2.0, 1.0), (-3.0, -0.5), (0.0, 2.0)):
                yield ta, tb, alpha, beta


def pin_ex_integer_library(lib):
    # Integer operands: the product is exact, so it must equal numpy's exact
    # int64 product of the transposed/untransposed operands, scaled and added.
    M, N, K = 13, 11, 17
    for t, (ta, tb, alpha, beta) in enumerate(_ex_cases()):
        A, B = make_operands(M, N, K, "int", seed=300 + t)
        A, B = as_numpy(A), as_numpy(B)
        C0 = as_numpy(make_operands(M, 1, N, "int", seed=400 + t)[0])  # an M x N integer matrix
        As = np.ascontiguousarray(A.T) if ta else A  # stored form
        Bs = np.ascontiguousarray(B.T) if tb else B
        got, S, E = oracle.sgemm_ex_f64(ta, tb, alpha, As, Bs, beta, C0, lib=lib)
        prod = np.matmul(A.astype(np.int64), B.astype(np.int64)).astype(np.float64)
        want = alpha * prod + beta * C0.astype(np.float64) if beta != 0 else alpha * prod
        if alpha == 0:
            want = beta * C0.astype(np.float64)
        assert np.array_equal(got, want), (ta, tb, alpha, beta)
        mag = np.matmul(np.abs(A.astype(np.int64)), np.abs(B.astype(np.int64))).astype(np.float64)
        assert np.array_equal(S, abs(alpha) * mag if alpha != 0 else np.zeros_like(mag)), "S"
        assert np.array_equal(E, np.abs(want - (beta * C0 if beta != 0 else 0)) + np.abs(beta * C0 if beta != 0 else 0)), "E"


def pin_ex_hand_transposed(lib):
    # op(A) = A^T with A stored 2 x 3 = [[1, 2, 3], [4, 5, 6]] -> op(A) 3 x 2;
    # op(B) = B^T with B stored 2 x 2 = [[1, 0], [1, 1]] -> op(B) = [[1, 1], [0, 1]].
    # op(A) op(B) = [[1, 1+4], [2, 2+5], [3, 3+6]] = [[1, 5], [2, 7], [3, 9]];
    # times alpha = 2, plus beta = 1 times C0 = ones: [[3, 11], [5, 15], [7, 19]].
    A = np.array([[1, 2, 3], [4, 5, 6]], np.float32)
    B = np.array([[1, 0], [1, 1]], np.float32)
    got, _, _ = oracle.sgemm_ex_f64(True, True, 2.0, A, B, 1.0, np.ones((3, 2), np.float32), lib=lib)
    assert np.array_equal(got, [[3, 11], [5, 15], [7, 19]]), got


def pin_ex_unread_operands(lib):
    # beta == 0: C0 is not read (NaN there does not propagate);
    # alpha == 0: A and B are not read.
    A, B = make_operands(5, 6, 7, "uniform", seed=500)
    A, B = as_numpy(A), as_numpy(B)
    nan_c = np.full((5, 6), np.nan, np.float32)
    got, _, _ = oracle.sgemm_ex_f64(False, False, 1.0, A, B, 0.0, nan_c, lib=lib)
    assert np.isfinite(got).all()
    nan_a = np.full((5, 7), np.nan, np.float32)
    nan_b = np.full((7, 6), np.nan, np.float32)
    C0 = np.arange(30, dtype=np.float32).reshape(5, 6)
    got, _, _ = oracle.sgemm_ex_f64(False, False, 0.0, nan_a, nan_b, 3.0, C0, lib=lib)
    assert np.array_equal(got, 3.0 * C0.astype(np.float64))


ALL_PINS += [pin_ex_integer_library, pin_ex_hand_transposed, pin_ex_unread_operands]
