"""Pins of the two parity measures every GPU comparison goes through.

The tolerances of the workloads are stated as a relative L2 distance
||y - ref||_2 / ||ref||_2 and a maximum absolute error max |y - ref|.  These
checks use pairs whose distances are worked out by hand (Pythagorean triples,
so every value is exact), chosen so that a swapped denominator, a missing
square root, a missing absolute value or a dropped element each fail one of
them.
"""
import numpy as np
import pytest

import oracle


def test_rel_l2_hand_worked_pair():
    # ref has norm 3 (1, 2, 2); the difference has norm 0.5 (0.3, 0.4)
    ref = np.array([1.0, -2.0, 2.0])
    y = ref + np.array([0.0, 0.3, -0.4])
    assert oracle.rel_l2(y, ref) == pytest.approx(0.5 / 3.0, rel=1e-15)
    # the denominator is the reference's norm, not y's: ||y|| = sqrt(1 + 1.7^2 + 1.6^2)
    assert oracle.rel_l2(ref, y) == pytest.approx(0.5 / np.sqrt(1 + 1.7 ** 2 + 1.6 ** 2), rel=1e-15)


def test_rel_l2_is_a_norm_not_a_sum_of_squares():
    # difference (3, 4) has norm 5; ref (0, 0, 12, 5) has norm 13
    ref = np.array([[0.0, 0.0], [12.0, 5.0]])
    y = ref + np.array([[3.0, 4.0], [0.0, 0.0]])
    assert oracle.rel_l2(y, ref) == pytest.approx(5.0 / 13.0, rel=1e-15)
    # every element counts, across all axes
    y2 = ref.copy()
    y2[1, 1] += 13.0
    assert oracle.rel_l2(y2, ref) == pytest.approx(1.0, rel=1e-15)


def test_rel_l2_equal_and_zero_reference():
    a = np.arange(12.0).reshape(3, 4)
    assert oracle.rel_l2(a, a) == 0.0
    # an all-zero reference has no scale: the plain norm of y is returned
    assert oracle.rel_l2(np.array([3.0, 4.0]), np.zeros(2)) == pytest.approx(5.0, rel=1e-15)


def test_max_abs_hand_worked_pair():
    ref = np.array([1.0, -2.0, 2.0])
    # the largest deviation is negative: without the absolute value it would read 0.3
    y = ref + np.array([0.0, 0.3, -0.4])
    assert oracle.max_abs(y, ref) == pytest.approx(0.4, rel=1e-15)
    assert oracle.max_abs(ref, y) == pytest.approx(0.4, rel=1e-15)
    # every element and axis counts
    m = np.zeros((2, 3, 4))
    m2 = m.copy()
    m2[1, 2, 3] = -7.5
    assert oracle.max_abs(m2, m) == 7.5
    assert oracle.max_abs(m, m) == 0.0
    assert oracle.max_abs(np.zeros(0), np.zeros(0)) == 0.0
