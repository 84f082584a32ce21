"""The result checker against its pins, and the pins against broken checkers."""
import importlib.util
import os

import pytest

from oracle import check
from tests import checker_pins


@pytest.mark.parametrize("pin", checker_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(check)


def test_page_relative_error_formula():
    # max |g - r| / max(|r|, 1e-6), the figure the course's checker prints.
    import numpy as np
    r = check.check(np.array([1.5, 0.0], np.float32), np.array([1.0, 0.0]), np.array([10.0, 1.0]), 1 << 20)
    assert r["max_rel_err_page"] == pytest.approx(0.5)


def test_shape_mismatch_raises():
    import numpy as np
    with pytest.raises(ValueError):
        check.check_ex(np.zeros((2, 3)), np.zeros((3, 2)), np.zeros((3, 2)), np.zeros((3, 2)), 1)


# Plausible mistakes in the checker; each must make some pin fail.  The
# too-loose ones matter most: they would let wrong GPU results pass.
MUTANTS = {
    "drop_E": ("return bound(S, K) + SLACK_E * U * np.asarray(E, dtype=np.float64)",
               "return bound(S, K)"),
    "swap_S_E": ("return bound(S, K) + SLACK_E * U * np.asarray(E, dtype=np.float64)",
                 "return bound(E, K) + SLACK_E * U * np.asarray(S, dtype=np.float64)"),
    "E_slack_4": ("SLACK_E = 2.0", "SLACK_E = 4.0"),
    "E_slack_1": ("SLACK_E = 2.0", "SLACK_E = 1.0"),
    "slack_8": ("SLACK = 4.0", "SLACK = 8.0"),
    "slack_2": ("SLACK = 4.0", "SLACK = 2.0"),
    "u_2_23": ("U = 2.0 ** -24", "U = 2.0 ** -23"),
    "k_plus_1": ("SLACK * K * U", "SLACK * (K + 1) * U"),
    "k_squared": ("SLACK * K * U", "SLACK * K * K * U"),
    "signed_error": ("err = np.abs(g - r)", "err = g - r"),
    "nan_only": ("bad = ~np.isfinite(g)", "bad = np.isnan(g)"),
    "no_nonfinite_check": ("viol = bad | (err > b)", "viol = err > b"),
    "non_strict": ("viol = bad | (err > b)", "viol = bad | (err >= b)"),
    "relative_gate": ("viol = bad | (err > b)", "viol = bad | (err > b * np.maximum(np.abs(r), 1.0))"),
}


def _load_mutant(tmp_path, name):
    src = open(check.__file__).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    path = tmp_path / f"check_{name}.py"
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location(f"check_{name}", str(path))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_checker_mutant(tmp_path, name):
    mod = _load_mutant(tmp_path, name)
    caught = []
    for pin in checker_pins.ALL_PINS:
        try:
            pin(mod)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin caught checker mutant {name}"
    assert os.path.exists(check.__file__)
