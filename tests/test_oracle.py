"""The CPU oracle against its pins, and the pins against broken oracles."""
import os
import re
import subprocess
import sys

import numpy as np
import pytest

import oracle
from oracle import check
from tests import oracle_pins
from roofline_sgemm_f32_amd.inputs import as_numpy, make_operands


@pytest.fixture(scope="module")
def lib():
    oracle.build(force=False)
    return oracle.load()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(lib, pin):
    pin(lib)


def test_thread_count_does_not_change_result(lib):
    A, B = make_operands(67, 45, 129, "normal", seed=3)
    A, B = as_numpy(A), as_numpy(B)
    c1, s1 = oracle.sgemm_f64(A, B, threads=1)
    c7, s7 = oracle.sgemm_f64(A, B, threads=7)
    assert np.array_equal(c1, c7) and np.array_equal(s1, s7)


def test_entry_points_agree_bitwise(lib):
    A, B = make_operands(33, 70, 91, "uniform", seed=4, lda=95, ldb=70)
    A, B = as_numpy(A), as_numpy(B)
    C, S = oracle.sgemm_f64(A, B)
    rows = np.array([32, 0, 17])
    R, RS = oracle.sgemm_rows_f64(A, B, rows)
    assert np.array_equal(R, C[rows]) and np.array_equal(RS, S[rows])
    ii = np.array([0, 5, 32, 32]), np.array([69, 0, 1, 69])
    E, ES = oracle.sgemm_entries_f64(A, B, *ii)
    assert np.array_equal(E, C[ii]) and np.array_equal(ES, S[ii])


# --- the checker -----------------------------------------------------------

def test_checker_accepts_float_rounding_and_rejects_errors():
    A, B = make_operands(20, 30, 500, "uniform", seed=5)
    A, B = as_numpy(A), as_numpy(B)
    C, S = oracle.sgemm_f64(A, B)
    # float32 accumulation in ascending k: a correct float result.
    f = np.zeros((20, 30), dtype=np.float32)
    for k in range(500):
        f = (f + np.outer(A[:, k], B[k, :]).astype(np.float32)).astype(np.float32)
    rep = check.check(f, C, S, 500)
    assert rep["ok"] and rep["max_bound_util"] < 1.0
    bad = f.copy()
    bad[3, 4] += 0.5  # far outside the bound (about 0.015 here)
    assert not check.check(bad, C, S, 500)["ok"]
    nan = f.copy()
    nan[0, 0] = np.nan
    r = check.check(nan, C, S, 500)
    assert not r["ok"] and r["n_nonfinite"] == 1


# --- mutation: each plausible mistake in the oracle must trip a pin ---------

MUTANTS = {
    "drop_last_k": ("for (int64_t k = 0; k < K; k++) {\n        const double aik",
                    "for (int64_t k = 0; k < K - 1; k++) {\n        const double aik"),
    "wrong_sign": ("acc[j] += aik * (double)brow[j];", "acc[j] -= aik * (double)brow[j];"),
    "transposed_b": ("acc[j] += aik * (double)brow[j];", "acc[j] += aik * (double)B[j * ldb + k];"),
    "lda_as_k": ("j->A + src * j->lda", "j->A + src * j->K"),
    "float_products": ("acc[j] += aik * (double)brow[j];", "acc[j] += (double)(float)(aik * (double)brow[j]);"),
    "row_off_by_one": ("const int64_t src = j->rows ? j->rows[r] : r;",
                       "const int64_t src = j->rows ? j->rows[r] : (r + 1) % (j->r1 > 0 ? j->r1 : 1);"),
    "entries_b_stride": ("(double)b[k * ldb]", "(double)b[k * (ldb - 1)]"),
    "bound_signed": ("s[j] += mag * fabs((double)brow[j]);", "s[j] += aik * (double)brow[j];"),
    "entries_drop_first": ("for (int64_t k = 0; k < K; k++) {\n            const double p",
                           "for (int64_t k = 1; k < K; k++) {\n            const double p"),
    "chain_unfused": ("acc = fmaf(acc, x, y);", "acc = acc * x; acc = acc + y;"),
    "chain_start": ("float acc = 0.0625f * (float)(j + 1);", "float acc = 0.0625f * (float)j;"),
    "probe_transposed": ("(double)a_vals[i + 32 * k] * (double)b_vals[j + 32 * k]",
                         "(double)a_vals[32 * i % 64 + k] * (double)b_vals[j + 32 * k]"),
    "probe_one_k": ("for (int k = 0; k < 2; k++) p +=", "for (int k = 0; k < 1; k++) p +="),
    "ex_transa_index": ("transa ? (double)A[k * lda + i]", "transa ? (double)A[i * lda + k]"),
    "ex_transb_index": ("transb ? (double)B[j * ldb + k]", "transb ? (double)B[k * ldb + j]"),
    "ex_beta_dropped": ("const double c0 = beta != 0.0 ? beta * (double)C0[i * ldc0 + j] : 0.0;",
                        "const double c0 = 0.0;"),
    "ex_alpha_on_c0": ("C[i * ldc + j] = alpha * acc + c0;", "C[i * ldc + j] = alpha * (acc + c0);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(tmp_path, name):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mutated = tmp_path / "oracle_mut.c"
    mutated.write_text(src.replace(old, new))
    so = tmp_path / "liboracle_mut.so"
    subprocess.check_call(["gcc", *oracle.CFLAGS, str(mutated), "-o", str(so), "-lm"])
    # Run the pins in a child process: a mutant that reads out of bounds may
    # crash, which also counts as caught.
    code = (
        "import sys, oracle\n"
        "from tests import oracle_pins\n"
        f"lib = oracle.load({str(so)!r})\n"
        "caught = []\n"
        "for pin in oracle_pins.ALL_PINS:\n"
        "    try:\n"
        "        pin(lib)\n"
        "    except (AssertionError, IndexError, ValueError):\n"
        "        caught.append(pin.__name__)\n"
        "print('CAUGHT', ' '.join(caught))\n"
        "sys.exit(0 if caught else 3)\n"
    )
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    res = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True,
                         timeout=300)
    assert res.returncode != 3, f"no pin caught mutant {name}: {res.stdout}{res.stderr}"
