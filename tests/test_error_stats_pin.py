"""Pins of the acceptance metric every GPU parity assertion applies.

The bar for floating-point outputs is max|err| <= 1e-2 * max|ref| and a
relative L2 error <= 5e-3.  `error_stats` turns a (got, ref) pair into those
two ratios; each case below is worked by hand, and each is chosen so that a
plausible slip fails it: dividing by max|got| instead of max|ref|, squaring the
norms, dropping the absolute value, taking a mean instead of a maximum, or
letting an all-zero reference pass any output."""
from __future__ import annotations

import math

import numpy as np
import pytest

from oracle.gqla_ref import error_stats


def test_three_element_case_worked_by_hand():
    # err = (0, 0, -1): max|err| = 1, max|ref| = 4; ||err|| = 1, ||ref|| = sqrt(1 + 4 + 16)
    st = error_stats([1.0, 2.0, 3.0], [1.0, 2.0, 4.0])
    assert st["max_err"] == 1.0 and st["max_ref"] == 4.0
    assert st["max_rel"] == 0.25
    assert st["rel_l2"] == pytest.approx(1.0 / math.sqrt(21.0), rel=1e-15)
    assert st["finite"]


def test_max_rel_divides_by_the_reference_maximum_not_the_output_maximum():
    # max|got| = 10 differs from max|ref| = 2: 8 / 2 = 4 (8 / 10 would be the slip)
    st = error_stats([10.0, 0.0], [2.0, 0.0])
    assert st["max_rel"] == 4.0


def test_rel_l2_is_a_ratio_of_unsquared_norms():
    # err = (3, -4): ||err|| = 5, ||ref|| = 4 -> 1.25 (squared norms would give 25 / 16)
    st = error_stats([3.0, 0.0], [0.0, 4.0])
    assert st["rel_l2"] == 1.25
    assert st["max_rel"] == 1.0          # max|err| = 4, max|ref| = 4


def test_magnitudes_not_signed_values():
    # ref (-5, 1): max|ref| = 5 although max(ref) = 1; err (1, 0) -> 1 / 5
    st = error_stats([-4.0, 1.0], [-5.0, 1.0])
    assert st["max_rel"] == pytest.approx(0.2, rel=1e-15)
    assert st["rel_l2"] == pytest.approx(1.0 / math.sqrt(26.0), rel=1e-15)


def test_maximum_not_mean_of_the_error():
    # one large error among many zeros: max|err| = 3 over max|ref| = 1
    ref = np.ones(1000)
    got = ref.copy()
    got[417] += 3.0
    st = error_stats(got, ref)
    assert st["max_rel"] == 3.0
    assert st["rel_l2"] == pytest.approx(3.0 / math.sqrt(1000.0), rel=1e-14)


def test_all_zero_reference_admits_only_an_exact_zero():
    z = np.zeros((2, 3))
    st = error_stats(z, z)
    assert st["max_rel"] == 0.0 and st["rel_l2"] == 0.0
    got = z.copy()
    got[1, 2] = 1e-30
    st = error_stats(got, z)
    assert st["max_rel"] == math.inf and st["rel_l2"] == math.inf


def test_non_finite_output_is_flagged_and_fails_the_bar():
    st = error_stats([1.0, float("nan")], [1.0, 1.0])
    assert not st["finite"]
    assert not (st["max_rel"] <= 1e-2)          # NaN compares false
    st = error_stats([1.0, float("inf")], [1.0, 1.0])
    assert not st["finite"] and st["max_rel"] == math.inf


def test_the_bar_applied_to_a_uniform_relative_perturbation():
    # got = ref * (1 + e) with |e| = 1e-3 everywhere: both ratios equal 1e-3
    rng = np.random.default_rng(3)
    ref = rng.standard_normal(4096)
    got = ref * (1.0 + 1e-3)
    st = error_stats(got, ref)
    assert st["max_rel"] == pytest.approx(1e-3, rel=1e-9)
    assert st["rel_l2"] == pytest.approx(1e-3, rel=1e-9)


def test_shapes_must_agree():
    with pytest.raises(ValueError):
        error_stats(np.zeros(3), np.zeros(4))
