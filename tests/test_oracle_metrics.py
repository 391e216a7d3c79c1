"""Pins of the parity gate itself (oracle.metrics), on values worked out by
hand: a known ratio, the zero-scale branch (equal and unequal values), a
non-finite result, a shape mismatch and an empty array.  If any branch were
wrong every GPU parity test could pass without checking anything.  CPU only.

The gate is the reading of "max relative error 1e-5" (and the pages' float64
comparisons at 1e-12, cuequivariance-torch skill document, "Spherical
harmonics and a NumPy reference" and "Channelwise product with external
per-example weights") as an error scaled by the sum of absolute terms."""

import math

import numpy as np
import pytest

from oracle import metrics


def test_known_ratio():
    # |1.5 - 1| / 2 = 0.25, |-2 - (-2.5)| / 10 = 0.05, |0 - 0| / 3 = 0: max 0.25
    got = np.array([1.5, -2.0, 0.0])
    ref = np.array([1.0, -2.5, 0.0])
    scale = np.array([2.0, 10.0, 3.0])
    assert metrics.scaled_error(got, ref, scale) == 0.25


def test_ratio_is_per_element_not_global():
    # the small-scale element decides: 1e-3 / 1e-2 = 0.1 beats 1 / 100 = 0.01
    got = np.array([101.0, 0.011])
    ref = np.array([100.0, 0.010])
    scale = np.array([100.0, 0.01])
    assert math.isclose(metrics.scaled_error(got, ref, scale), 0.1, rel_tol=1e-12)


def test_exact_match_is_zero():
    a = np.array([[1.0, -3.0], [7.25, 0.0]])
    assert metrics.scaled_error(a, a.copy(), np.abs(a) + 1) == 0.0


def test_zero_scale_equal_values_pass():
    # A_i = 0 means every term of the sum is zero: the result must be exactly 0
    got = np.array([0.0, 1.0])
    ref = np.array([0.0, 1.0])
    scale = np.array([0.0, 1.0])
    assert metrics.scaled_error(got, ref, scale) == 0.0


def test_zero_scale_unequal_values_fail():
    got = np.array([1e-30, 1.0])
    ref = np.array([0.0, 1.0])
    scale = np.array([0.0, 1.0])
    assert metrics.scaled_error(got, ref, scale) == math.inf


def test_zero_scale_negative_zero_is_equal():
    assert metrics.scaled_error(np.array([-0.0]), np.array([0.0]), np.array([0.0])) == 0.0


@pytest.mark.parametrize("bad", [math.nan, math.inf, -math.inf])
def test_non_finite_result_fails(bad):
    got = np.array([1.0, bad])
    ref = np.array([1.0, 2.0])
    scale = np.array([1.0, 1e300])
    assert metrics.scaled_error(got, ref, scale) == math.inf


def test_nan_where_scale_is_zero_fails():
    assert metrics.scaled_error(np.array([math.nan]), np.array([0.0]), np.array([0.0])) == math.inf


@pytest.mark.parametrize("shapes", [((3,), (3,), (4,)), ((3,), (1, 3), (3,)), ((2, 3), (3, 2), (2, 3))])
def test_shape_mismatch_raises(shapes):
    a, b, c = (np.ones(s) for s in shapes)
    with pytest.raises(ValueError):
        metrics.scaled_error(a, b, c)


def test_empty_is_zero():
    e = np.zeros((0, 5))
    assert metrics.scaled_error(e, e, e) == 0.0


def test_accepts_float32_input_exactly():
    # float32 values are widened exactly before the subtraction
    got = np.array([np.float32(1.0) + np.float32(2.0 ** -23)], dtype=np.float32)
    assert metrics.scaled_error(got, np.array([1.0]), np.array([1.0])) == 2.0 ** -23


def test_normwise_known_ratio():
    # max |got - ref| = 0.5, max |ref| = 4
    got = np.array([1.0, -4.5, 2.0])
    ref = np.array([1.0, -4.0, 2.25])
    assert metrics.normwise_error(got, ref) == 0.125


def test_normwise_zero_reference_and_empty():
    assert metrics.normwise_error(np.array([0.0, -3.0]), np.zeros(2)) == 3.0
    assert metrics.normwise_error(np.zeros(0), np.zeros(0)) == 0.0
