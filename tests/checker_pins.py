"""Pins for the oracle's checkers (CPU only).

Every GPU verdict goes through three functions of the oracle package:
``error_bound`` (the element-wise tolerance), ``check_within_bound`` (the test
for real-valued inputs) and ``check_bitexact`` (the test for integer-valued
inputs).  These pins hold them to values worked out by hand, so that a slip in
any of them (a wrong factor, a dropped term, a strict comparison, a NaN that
passes, a comparison of values instead of bit patterns) fails a pin instead of
passing every GPU test silently.

The tolerance is the one the product is held to:

    |C - Cref| <= 2e-5 * (|alpha| * (|A|*|B|)_ij + |beta| * |C0_ij|)

with the C0 term absent when beta == 0 (C0 is then not read, so it may hold
NaN).  Each pin takes an object ``k`` with the three functions, so that the
same pins run against copies of the package with a planted mistake.
"""
from __future__ import annotations

import numpy as np


def _f32(*v):
    return np.array(v, dtype=np.float32)


def cpin_bound_two_terms(k):
    # alpha = -1.5, beta = -0.5: both terms count with their magnitudes.
    absab = np.array([[2.0, 4.0], [0.0, 10.0]])
    C0 = np.array([[-6.0, 8.0], [3.0, -0.0]], np.float32)
    got = k.error_bound(absab, -1.5, -0.5, C0)
    # 1.5*2 + 0.5*6 = 6; 1.5*4 + 0.5*8 = 10; 0 + 0.5*3 = 1.5; 1.5*10 + 0 = 15
    want = np.array([[6.0, 10.0], [1.5, 15.0]]) * 2e-5
    assert got.shape == (2, 2)
    assert np.allclose(got, want, rtol=1e-12, atol=0), (got, want)


def cpin_bound_beta_zero_ignores_c0(k):
    absab = np.array([1.0, 3.0, 0.5])
    nanC = _f32(np.nan, np.inf, -7.0)
    got = k.error_bound(absab, 2.0, 0.0, nanC)
    assert np.all(np.isfinite(got)), got
    assert np.allclose(got, 2e-5 * 2.0 * absab, rtol=1e-12, atol=0), got
    got = k.error_bound(absab, 2.0, 0.0, None)
    assert np.allclose(got, 2e-5 * 2.0 * absab, rtol=1e-12, atol=0), got


def cpin_bound_alpha_only_when_no_product(k):
    # alpha = 0: only the C0 term is left (|A||B| is zero for such calls).
    got = k.error_bound(np.zeros(3), 0.0, 4.0, _f32(1.0, -2.0, 0.25))
    assert np.allclose(got, 2e-5 * 4.0 * np.array([1.0, 2.0, 0.25]), rtol=1e-12, atol=0), got


def cpin_bound_scalars_as_float32(k):
    # The scalars enter the product as float32 values: 0.1 is 0.100000001490116...
    got = k.error_bound(np.array([1.0]), 0.1, 0.0, None)
    want = 2e-5 * float(np.float32(0.1))
    assert abs(got[0] - want) <= 1e-12 * want and got[0] != 2e-5 * 0.1, (got, want)


def cpin_within_bound_edges(k):
    # err exactly at the bound passes; one float32 step beyond it fails, on
    # either side of Cref.
    Cref = np.array([1.0, 1.0, 1.0])
    bound = np.full(3, 2.0 ** -10)
    at = _f32(1 + 2.0 ** -10, 1 - 2.0 ** -10, 1.0)
    ok, info = k.check_within_bound(at, Cref, bound)
    assert ok and info["n_bad"] == 0, info
    assert info["max_err_over_bound"] == 1.0, info
    above = _f32(1.0, 1 + 2.0 ** -10 + 2.0 ** -23, 1.0)
    ok, info = k.check_within_bound(above, Cref, bound)
    assert not ok and info["n_bad"] == 1 and info["first_bad_index"] == (1,), info
    below = _f32(1.0, 1.0, 1 - 2.0 ** -10 - 2.0 ** -24)
    ok, info = k.check_within_bound(below, Cref, bound)
    assert not ok and info["n_bad"] == 1 and info["first_bad_index"] == (2,), info


def cpin_within_bound_zero_bound(k):
    # A zero bound (an all-zero row of A, beta = 0) admits only an exact zero.
    Cref = np.zeros(2)
    bound = np.zeros(2)
    ok, _ = k.check_within_bound(_f32(0.0, -0.0), Cref, bound)
    assert ok
    ok, info = k.check_within_bound(_f32(0.0, 1e-30), Cref, bound)
    assert not ok and info["n_bad"] == 1, info


def cpin_within_bound_nonfinite(k):
    Cref = np.array([[3.0, -2.0], [0.5, 7.0]])
    bound = np.full((2, 2), 1.0)
    for bad_val, where in ((np.nan, (0, 1)), (np.inf, (1, 0)), (-np.inf, (1, 1))):
        C = Cref.astype(np.float32)
        C[where] = bad_val
        ok, info = k.check_within_bound(C, Cref, bound)
        assert not ok and info["n_bad"] == 1, (bad_val, info)
        assert info["first_bad_index"] == where, (bad_val, info)


def cpin_within_bound_counts(k):
    rng = np.random.default_rng(3)
    Cref = rng.standard_normal((5, 7))
    bound = np.full((5, 7), 0.5)
    C = Cref.astype(np.float32)
    C[1, 2] += 0.75
    C[3, 6] -= 2.0
    C[4, 0] += 0.25
    ok, info = k.check_within_bound(C, Cref, bound)
    assert not ok and info["n_bad"] == 2 and info["first_bad_index"] == (1, 2), info
    assert abs(info["max_err_over_bound"] - 4.0) < 1e-5, info


def cpin_bitexact(k):
    Cref = np.array([1.0, -3.5, 1 + 2.0 ** -30, 65536.0])
    # float32(1 + 2^-30) is 1.0: the reference is rounded to float32 first.
    ok, info = k.check_bitexact(_f32(1.0, -3.5, 1.0, 65536.0), Cref)
    assert ok and info["n_bad"] == 0, info
    ok, info = k.check_bitexact(_f32(1.0, -3.5, 1.0 + 2.0 ** -23, 65536.0), Cref)
    assert not ok and info["n_bad"] == 1 and info["first_bad_index"] == (2,), info
    ok, info = k.check_bitexact(_f32(1.0, -3.5, 1.0, 65540.0), Cref)
    assert not ok and info["first_bad_index"] == (3,), info


def cpin_bitexact_signed_zero_and_nan(k):
    # Bit patterns, not values: -0.0 differs from +0.0, and NaN never matches a number.
    ok, info = k.check_bitexact(_f32(-0.0, 2.0), np.array([0.0, 2.0]))
    assert not ok and info["first_bad_index"] == (0,), info
    ok, _ = k.check_bitexact(_f32(-0.0, 2.0), np.array([-0.0, 2.0]))
    assert ok
    ok, info = k.check_bitexact(_f32(1.0, np.nan), np.array([1.0, 4.0]))
    assert not ok and info["first_bad_index"] == (1,), info


CHECKER_PINS = [cpin_bound_two_terms, cpin_bound_beta_zero_ignores_c0,
                cpin_bound_alpha_only_when_no_product, cpin_bound_scalars_as_float32,
                cpin_within_bound_edges, cpin_within_bound_zero_bound,
                cpin_within_bound_nonfinite, cpin_within_bound_counts, cpin_bitexact,
                cpin_bitexact_signed_zero_and_nan]
