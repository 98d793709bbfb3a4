"""The oracle's checkers against their pins, and planted mistakes that the pins
must catch (CPU only).

A mutant is a copy of the oracle package's source with one plausible slip,
loaded as a separate module from a temporary directory; the real package is
untouched.
"""
import importlib.util

import pytest

from checker_pins import CHECKER_PINS


@pytest.mark.parametrize("pin", CHECKER_PINS, ids=[p.__name__ for p in CHECKER_PINS])
def test_checker_pin(oracle_mod, pin):
    pin(oracle_mod)


CHECKER_MUTATIONS = {
    "rel_tol_times_10": ("REL_TOL = 2e-5", "REL_TOL = 2e-4"),
    "rel_tol_over_10": ("REL_TOL = 2e-5", "REL_TOL = 2e-6"),
    "bound_drops_beta_term": ("bound = bound + abs(float(np.float32(beta))) * np.abs(",
                              "bound = bound + 0.0 * np.abs("),
    "bound_signed_alpha": ("bound = abs(float(np.float32(alpha))) * np.asarray",
                           "bound = float(np.float32(alpha)) * np.asarray"),
    "bound_signed_beta": ("bound = bound + abs(float(np.float32(beta))) * np.abs(",
                          "bound = bound + float(np.float32(beta)) * np.abs("),
    "bound_signed_c0": ("* np.abs(\n            np.asarray(c0_vals, dtype=np.float64))",
                        "* (\n            np.asarray(c0_vals, dtype=np.float64))"),
    "bound_reads_c0_when_beta_zero": ("if np.float32(beta) != 0 and c0_vals is not None:",
                                      "if c0_vals is not None:"),
    "bound_scalars_in_float64": ("bound = abs(float(np.float32(alpha))) * np.asarray",
                                 "bound = abs(float(alpha)) * np.asarray"),
    "strict_comparison": ("bad = ~(err <= bound)", "bad = ~(err < bound)"),
    "nan_passes": ("bad = ~(err <= bound)", "bad = err > bound"),
    "signed_error": ("err = np.abs(C64 - Cref)", "err = C64 - Cref"),
    "bitexact_by_value": ("diff = got.view(np.uint32) != want.view(np.uint32)",
                          "diff = got != want"),
    "bitexact_unrounded_reference": ("diff = got.view(np.uint32) != want.view(np.uint32)",
                                     "diff = got.astype(np.float64) != np.asarray(Cref)"),
}


def _load_mutant(oracle_mod, tmp_path, name):
    old, new = CHECKER_MUTATIONS[name]
    src = open(oracle_mod.__file__).read()
    assert src.count(old) == 1, f"mutation {name} does not apply to exactly one place"
    path = tmp_path / f"checker_mut_{name}.py"
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location(f"checker_mut_{name}", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name", sorted(CHECKER_MUTATIONS))
def test_checker_pins_catch_planted_mistake(oracle_mod, tmp_path, name):
    mutant = _load_mutant(oracle_mod, tmp_path, name)
    caught = []
    for pin in CHECKER_PINS:
        try:
            pin(mutant)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no checker pin caught mutation {name}"
