"""Pins of the two error measures every parity verdict goes through.

rel_l2 is ||x - y||_2 / ||y||_2 over the whole tensor and max_rel is the normwise
||x - y||_inf / ||y||_inf (the readings of "rel-L2" and "max-rel" taken for the
tolerances); the expected values below are worked out by hand, so a swapped
argument, a per-row norm or an elementwise maximum fails one of them.
"""
import math

import numpy as np

from oracle.metrics import max_rel, rel_l2


def test_rel_l2_hand_values():
    # diff = (0, 0, -1), ||y|| = sqrt(1 + 4 + 9)
    assert math.isclose(rel_l2([1.0, 2.0, 2.0], [1.0, 2.0, 3.0]), 1.0 / math.sqrt(14.0), rel_tol=1e-15)
    # diff = (0, 1), ||y|| = sqrt(2)
    assert math.isclose(rel_l2([1.0, 2.0], [1.0, 1.0]), 1.0 / math.sqrt(2.0), rel_tol=1e-15)


def test_rel_l2_divides_by_the_reference():
    # swapping the arguments changes the denominator: ||(1, 2, 2)|| = 3
    assert math.isclose(rel_l2([1.0, 2.0, 3.0], [1.0, 2.0, 2.0]), 1.0 / 3.0, rel_tol=1e-15)


def test_rel_l2_is_one_norm_over_the_whole_tensor():
    # rows are not normalised separately: diff = (1, 0, 0, -2) -> sqrt(5); ||y|| = 2
    x = np.array([[1.0, 0.0], [0.0, 0.0]])
    y = np.array([[0.0, 0.0], [0.0, 2.0]])
    assert math.isclose(rel_l2(x, y), math.sqrt(5.0) / 2.0, rel_tol=1e-15)


def test_max_rel_hand_values():
    assert max_rel([1.0, 2.0], [1.0, 1.0]) == 1.0
    # largest |diff| is 0.5 (second entry), largest |y| is 4
    assert max_rel([1.0, 2.5, -4.0], [1.0, 2.0, -4.0]) == 0.125


def test_max_rel_is_normwise_not_elementwise():
    # the small entry is off by half of itself; normwise that is 5e-4 of ||y||_inf,
    # elementwise it would be 0.5
    x = np.array([1.0, 0.0015])
    y = np.array([1.0, 0.001])
    assert math.isclose(max_rel(x, y), 5e-4, rel_tol=1e-12)
    # and the denominator is the reference's maximum, not the result's
    assert math.isclose(max_rel([0.0, 3.0], [0.0, 1.0]), 2.0, rel_tol=1e-15)


def test_zero_reference_and_empty():
    z = np.zeros(3)
    assert rel_l2(z, z) == 0.0 and max_rel(z, z) == 0.0
    assert rel_l2([0.0, 1e-30, 0.0], z) == math.inf
    assert max_rel([0.0, 1e-30, 0.0], z) == math.inf
    assert max_rel(np.zeros(0), np.zeros(0)) == 0.0
    assert rel_l2(np.zeros(0), np.zeros(0)) == 0.0


def test_float64_accumulation():
    # float32 inputs are compared in float64: a 1e-9 relative difference survives
    y = np.full(1000, 1.0, dtype=np.float64)
    x = y * (1.0 + 1e-9)
    assert math.isclose(rel_l2(x, y), 1e-9, rel_tol=1e-6)
