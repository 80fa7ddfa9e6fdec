"""Pins of the oracle's Newton-Schulz against the mathematics that fixes it.

An odd matrix polynomial acts on the singular values: with X = U S V^T and
p(s) = a s + b s^3 + c s^5, one quintic round maps X to U p(S) V^T.  So the
five rounds after the Frobenius scaling equal U p5(S / (||X||_F + eps)) V^T
(p5 = p applied five times), computed here from numpy's SVD and a scalar
evaluation of p.  A dropped term, a sign, a transposed operand, a wrong
orientation for tall slots, a wrong norm or a wrong step count all break it.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import frobenius_prescale, newton_schulz
from tests.conftest import GOLDEN

COEF = json.load(open(os.path.join(GOLDEN, "ns_coefficients.json")))
A, B, C, STEPS = COEF["a"], COEF["b"], COEF["c"], COEF["steps"]
EPS = 1e-7


def p_scalar(s):
    return A * s + B * s ** 3 + C * s ** 5


def p5(s, steps=STEPS):
    for _ in range(steps):
        s = p_scalar(s)
    return s


def closed_form(x):
    u, s, vt = np.linalg.svd(x, full_matrices=False)
    return (u * p5(s / (np.linalg.norm(x) + EPS))) @ vt


SHAPES = [(8, 8), (16, 4), (4, 16), (1, 12), (6, 12), (12, 6), (3, 40), (40, 3), (33, 17)]


@pytest.mark.parametrize("shape", SHAPES)
def test_ns_equals_svd_closed_form(shape):
    rng = np.random.default_rng(sum(shape))
    x = rng.normal(0, 1, (3,) + shape)
    got = newton_schulz(x, STEPS, A, B, C, EPS)
    for i in range(3):
        np.testing.assert_allclose(got[i], closed_form(x[i]), rtol=0, atol=1e-10)


def test_step_count_and_coefficients_matter():
    """The closed form separates 4 from 5 rounds and catches a sign flip of b."""
    rng = np.random.default_rng(0)
    x = rng.normal(0, 1, (1, 8, 8))
    ref = closed_form(x[0])
    assert np.abs(newton_schulz(x, 4, A, B, C, EPS)[0] - ref).max() > 1e-3
    assert np.abs(newton_schulz(x, 5, A, -B, C, EPS)[0] - ref).max() > 1e-3


def test_one_row_slot_is_a_scaled_unit_vector():
    """1 x n (the smear gate): X X^T is the scalar ||X||^2, so the result is
    p5(||g|| / (||g|| + eps)) * g / ||g||, with p5 evaluated in exact rationals."""
    rng = np.random.default_rng(12)
    g = rng.normal(0, 1e-3, (1, 1, 12))
    nrm = float(np.linalg.norm(g))
    s = Fraction(nrm) / (Fraction(nrm) + Fraction(EPS))
    fa, fb, fc = Fraction(A), Fraction(B), Fraction(C)
    for _ in range(STEPS):
        s = fa * s + fb * s ** 3 + fc * s ** 5
    want = float(s) * g[0] / nrm
    np.testing.assert_allclose(newton_schulz(g)[0], want, rtol=1e-12, atol=0)


def test_p5_at_one():
    """p applied five times to 1: 0.7010, 1.11362, 0.72071, 1.08997, 0.69644."""
    s = Fraction(1)
    vals = []
    for _ in range(STEPS):
        s = Fraction(A) * s + Fraction(B) * s ** 3 + Fraction(C) * s ** 5
        vals.append(float(s))
    np.testing.assert_allclose(vals, [0.7010, 1.11362, 0.72071, 1.08997, 0.69644], atol=6e-6)
    x = np.zeros((1, 1, 5))
    x[0, 0, 2] = 1.0
    np.testing.assert_allclose(newton_schulz(x, eps=0.0)[0, 0, 2], vals[-1], rtol=1e-13)


def _band():
    """Range of p5 over scaled singular values in [0.1, 1] (dense scalar scan)."""
    s = np.linspace(0.1, 1.0, 200001)
    v = p5(s)
    return v.min(), v.max()


def test_band_for_well_conditioned_inputs():
    lo, hi = _band()
    assert 0.68 < lo < 0.683 and 1.134 < hi < 1.135
    rng = np.random.default_rng(21)
    for (r, c) in [(16, 16), (12, 24), (24, 12)]:
        m = min(r, c)
        for _ in range(4):
            q1, _ = np.linalg.qr(rng.normal(size=(r, m)))
            q2, _ = np.linalg.qr(rng.normal(size=(c, m)))
            s = rng.uniform(0.5, 1.0, m)
            x = (q1 * s) @ q2.T
            sv = np.linalg.svd(newton_schulz(x[None])[0], compute_uv=False)
            assert sv.min() >= lo - 1e-9 and sv.max() <= hi + 1e-9


def test_polar_direction():
    """For outputs with singular values in [L, U], the cosine to the polar factor
    U V^T is at least (L+U)/sqrt(2(L^2+U^2)) = 0.970."""
    lo, hi = _band()
    bound = (lo + hi) / np.sqrt(2 * (lo ** 2 + hi ** 2))
    assert bound > 0.969
    rng = np.random.default_rng(22)
    for _ in range(5):
        q1, _ = np.linalg.qr(rng.normal(size=(16, 16)))
        q2, _ = np.linalg.qr(rng.normal(size=(16, 16)))
        x = (q1 * rng.uniform(0.5, 1, 16)) @ q2.T
        y = newton_schulz(x[None])[0]
        u, _, vt = np.linalg.svd(x)
        polar = u @ vt
        cos = np.sum(y * polar) / (np.linalg.norm(y) * np.linalg.norm(polar))
        assert cos >= bound


def test_equivariances():
    rng = np.random.default_rng(23)
    x = rng.normal(0, 1, (1, 10, 14))
    y = newton_schulz(x)[0]
    # transpose: NS(X^T) = NS(X)^T (the tall path transposes internally)
    np.testing.assert_allclose(newton_schulz(x.transpose(0, 2, 1))[0], y.T, atol=1e-12)
    # orthogonal: NS(Q X R) = Q NS(X) R
    q, _ = np.linalg.qr(rng.normal(size=(10, 10)))
    r, _ = np.linalg.qr(rng.normal(size=(14, 14)))
    np.testing.assert_allclose(newton_schulz((q @ x[0] @ r)[None])[0], q @ y @ r, atol=1e-12)
    # positive scale (up to eps / ||X||)
    np.testing.assert_allclose(newton_schulz(37.0 * x)[0], y, atol=1e-7)
    # batch permutation
    xb = rng.normal(0, 1, (5, 6, 9))
    perm = rng.permutation(5)
    np.testing.assert_allclose(newton_schulz(xb[perm]), newton_schulz(xb)[perm], atol=1e-14)


def test_zero_slot_stays_zero():
    x = np.zeros((2, 12, 6))
    x[1] = np.random.default_rng(1).normal(size=(12, 6))
    y = newton_schulz(x)
    assert np.all(y[0] == 0.0)
    assert np.abs(y[1]).max() > 0.1


def test_frobenius_prescale_matches_library_norm():
    x = np.random.default_rng(2).normal(0, 3, (17, 29))
    np.testing.assert_allclose(frobenius_prescale(x, 0.0), x / np.linalg.norm(x, "fro"), rtol=1e-14)
    assert np.all(frobenius_prescale(np.zeros((3, 3))) == 0.0)


# ---------------------------------------------------------------------------
# per-round coefficient schedules
# ---------------------------------------------------------------------------
# With round t using p_t(s) = a_t s + b_t s^3 + c_t s^5, the rounds map the scaled
# singular values through the composition p_T o ... o p_1 (each round is an odd
# matrix polynomial, acting on singular values).

SCHEDULE = [(3.4445, -4.7750, 2.0315), (3.0, -3.2, 1.2), (2.0, -1.5, 0.5), (1.875, -1.25, 0.375),
            (1.5, -0.5, 0.0)]


def closed_form_schedule(x, schedule):
    u, s, vt = np.linalg.svd(x, full_matrices=False)
    s = s / (np.linalg.norm(x) + EPS)
    for (ra, rb, rc) in schedule:
        s = ra * s + rb * s ** 3 + rc * s ** 5
    return (u * s) @ vt


@pytest.mark.parametrize("shape", [(8, 8), (6, 12), (12, 6), (1, 12), (5, 20)])
def test_schedule_equals_composed_closed_form(shape):
    rng = np.random.default_rng(100 + sum(shape))
    x = rng.normal(0, 1, (2,) + shape)
    got = newton_schulz(x, eps=EPS, schedule=SCHEDULE)
    for i in range(2):
        np.testing.assert_allclose(got[i], closed_form_schedule(x[i], SCHEDULE), rtol=0, atol=1e-10)


def test_schedule_order_matters_and_constant_schedule_is_the_fixed_round():
    rng = np.random.default_rng(101)
    x = rng.normal(0, 1, (1, 9, 7))
    fwd = newton_schulz(x, eps=EPS, schedule=SCHEDULE)
    rev = newton_schulz(x, eps=EPS, schedule=SCHEDULE[::-1])
    assert np.abs(fwd - rev).max() > 1e-3
    np.testing.assert_array_equal(newton_schulz(x, 5, A, B, C, EPS, schedule=[(A, B, C)] * 5),
                                  newton_schulz(x, 5, A, B, C, EPS))


def test_identity_rounds_leave_x_unchanged():
    """(1, 0, 0) is the identity polynomial: appending such rounds changes nothing."""
    rng = np.random.default_rng(102)
    x = rng.normal(0, 1, (2, 6, 10))
    one = newton_schulz(x, 1, A, B, C, EPS)
    np.testing.assert_allclose(newton_schulz(x, eps=EPS, schedule=[(A, B, C), (1, 0, 0), (1, 0, 0)]), one,
                               rtol=0, atol=1e-15)


def test_one_row_slot_with_schedule_in_exact_rationals():
    rng = np.random.default_rng(103)
    g = rng.normal(0, 1e-3, (1, 1, 12))
    nrm = float(np.linalg.norm(g))
    s = Fraction(nrm) / (Fraction(nrm) + Fraction(EPS))
    for (ra, rb, rc) in SCHEDULE:
        s = Fraction(ra) * s + Fraction(rb) * s ** 3 + Fraction(rc) * s ** 5
    np.testing.assert_allclose(newton_schulz(g, schedule=SCHEDULE)[0], float(s) * g[0] / nrm, rtol=1e-12, atol=0)
