"""Pins of the oracle's group-relative advantage (two-pass variance) against
closed forms, invariants, a library variance and brute force."""
import math

import numpy as np
import pytest

import oracle


def test_pair_closed_form():
    """Two completions with rewards a, b: mean (a+b)/2, std |a-b|/2, so the
    advantages are +-(a-b)/2 / (|a-b|/2 + eps)."""
    a, b, eps = 0.9, 0.2, 1e-3
    A = oracle.group_advantage([a, b], 2, eps)
    h = (a - b) / 2
    assert A[0] == pytest.approx(h / (abs(h) + eps), rel=1e-15)
    assert A[1] == pytest.approx(-h / (abs(h) + eps), rel=1e-15)


def test_zero_mean_unit_variance_per_group():
    g = np.random.default_rng(2)
    r = g.standard_normal(8 * 6) * 3 + 5
    A = oracle.group_advantage(r, 8, 0.0).reshape(6, 8)
    np.testing.assert_allclose(A.sum(1), 0, atol=1e-12)
    np.testing.assert_allclose((A * A).mean(1), 1.0, rtol=1e-12)


def test_matches_library_population_variance():
    g = np.random.default_rng(4)
    r = g.standard_normal(16 * 5)
    A = oracle.group_advantage(r, 16, 1e-4).reshape(5, 16)
    R = r.reshape(5, 16)
    exp = (R - R.mean(1, keepdims=True)) / (R.std(1, ddof=0, keepdims=True) + 1e-4)
    np.testing.assert_allclose(A, exp, rtol=1e-12)


def test_shift_and_scale_invariant_without_eps():
    g = np.random.default_rng(6)
    r = g.random(4 * 7)
    A = oracle.group_advantage(r, 4, 0.0)
    B = oracle.group_advantage(2.5 * r - 11.0, 4, 0.0)
    np.testing.assert_allclose(A, B, rtol=1e-10, atol=1e-12)


def test_two_pass_survives_a_large_offset():
    """A large common offset: the one-pass E[r^2] - E[r]^2 loses the spread in
    fp64, the two-pass form keeps it."""
    r = 1e9 + np.array([0.0, 1.0, 2.0, 3.0])
    A = oracle.group_advantage(r, 4, 0.0)
    s = math.sqrt(1.25)
    np.testing.assert_allclose(A, np.array([-1.5, -0.5, 0.5, 1.5]) / s, rtol=1e-9)


def test_constant_group_and_singletons_give_zero():
    A = oracle.group_advantage([1.0, 1.0, 1.0, 0.0, 3.0, 7.0], 3, 1e-6)
    assert np.all(A[:3] == 0.0)
    assert np.all(oracle.group_advantage([2.0, 2.0], 2, 0.0) == 0.0)   # 0/0 taken as 0
    assert np.all(oracle.group_advantage([0.3, -2.0, 5.0], 1, 1e-6) == 0.0)


def test_without_std_scaling_is_mean_centred():
    r = np.array([1.0, 0.0, 0.0, 1.0, 1.0, 1.0])
    A = oracle.group_advantage(r, 3, 1e-6, scale_by_std=False)
    np.testing.assert_allclose(A, [2 / 3, -1 / 3, -1 / 3, 0, 0, 0], atol=1e-15)


def test_brute_force_tiny():
    r = [0.5, -1.0, 2.0, 0.0, 1.0, 1.5]
    A = oracle.group_advantage(r, 3, 0.01)
    for g0 in (0, 3):
        grp = r[g0:g0 + 3]
        m = (grp[0] + grp[1] + grp[2]) / 3
        v = ((grp[0] - m) ** 2 + (grp[1] - m) ** 2 + (grp[2] - m) ** 2) / 3
        for i in range(3):
            assert A[g0 + i] == pytest.approx((grp[i] - m) / (math.sqrt(v) + 0.01), rel=1e-14)


def test_bad_group_size():
    with pytest.raises(ValueError):
        oracle.group_advantage([1.0, 2.0, 3.0], 2, 0.0)
