"""Pins of the oracle's per-iteration (minimax) Newton-Schulz coefficients.

The oracle's Remez solver and schedule are tied to facts outside themselves:
the definition of the best approximation solved as a linear programme on a
dense grid (scipy), the alternation property, brute-force perturbation, the
closed-form limit polynomial, and the SVD closed form of the matrix
iteration with per-iteration rows.
"""
from fractions import Fraction

import numpy as np
import pytest
import scipy.optimize as so

import oracle as O

INTERVALS = [(1e-3, 1.0), (0.05, 1.3), (0.5, 1.5), (0.9, 1.12), (0.2, 0.21)]


def lp_best_quintic(lo, hi, n=20001):
    """min E s.t. |1 - (a x + b x^3 + c x^5)| <= E on n grid points (HiGHS)."""
    x = np.linspace(lo, hi, n)
    V = np.stack([x, x ** 3, x ** 5], axis=1)
    one = np.ones((n, 1))
    A_ub = np.vstack([np.hstack([-V, -one]), np.hstack([V, -one])])
    b_ub = np.concatenate([-np.ones(n), np.ones(n)])
    res = so.linprog([0, 0, 0, 1], A_ub=A_ub, b_ub=b_ub, bounds=[(None, None)] * 4,
                     method="highs")
    assert res.status == 0
    return res.x


@pytest.mark.parametrize("lo,hi", INTERVALS)
def test_minimax_matches_linear_programme(lo, hi):
    a, b, c, E = O.minimax_quintic(lo, hi)
    la, lb, lc, lE = lp_best_quintic(lo, hi)
    # the grid LP sees a subset of the interval: its E is at most the true E
    assert lE <= E * (1 + 1e-9) + 1e-15
    # HiGHS solves to ~1e-8 absolute; a narrow interval makes (a, b, c)
    # ill-conditioned, so the coefficients are compared more loosely there
    assert E - lE <= 5e-8 + 1e-6 * E
    np.testing.assert_allclose([a, b, c], [la, lb, lc], rtol=1e-4 if hi - lo < 0.1 else 1e-6)


@pytest.mark.parametrize("lo,hi", INTERVALS)
def test_minimax_alternates(lo, hi):
    coef = O.minimax_quintic(lo, hi)[:3]
    E = O.minimax_quintic(lo, hi)[3]
    x = np.linspace(lo, hi, 400001)
    err = 1.0 - O.quintic_eval(coef, x)
    assert np.max(np.abs(err)) == pytest.approx(E, rel=1e-9)
    # +E at lo, -E at hi, and both signs inside: four alternation points
    assert err[0] == pytest.approx(E, rel=1e-9)
    assert err[-1] == pytest.approx(-E, rel=1e-9)
    i1 = int(np.argmin(err[: len(x) // 2 + len(x) // 4]))
    assert err[i1] == pytest.approx(-E, rel=1e-6)
    assert np.max(err[i1:]) == pytest.approx(E, rel=1e-6)


@pytest.mark.parametrize("lo,hi", [(1e-3, 1.0), (0.5, 1.5)])
def test_minimax_not_improvable(lo, hi):
    a, b, c, E = O.minimax_quintic(lo, hi)
    x = np.linspace(lo, hi, 20001)
    rng = np.random.default_rng(7)
    for _ in range(300):
        d = rng.standard_normal(3)
        d *= 10.0 ** rng.uniform(-6, -2) / np.linalg.norm(d)
        trial = (a + d[0] * abs(a), b + d[1] * abs(b), c + d[2] * abs(c))
        assert np.max(np.abs(1.0 - O.quintic_eval(trial, x))) >= E * (1 - 1e-9)


def test_limit_polynomial_closed_form():
    a, b, c = (Fraction(15, 8), Fraction(-10, 8), Fraction(3, 8))
    assert (float(a), float(b), float(c)) == O.LIMIT_QUINTIC
    assert a + b + c == 1                 # p(1) = 1
    assert a + 3 * b + 5 * c == 0         # p'(1) = 0
    assert 6 * b + 20 * c == 0            # p''(1) = 0
    # p'(x) = (15/8) (1 - x^2)^2 >= 0: increasing everywhere
    x = np.linspace(-2, 2, 1001)
    deriv = float(a) + 3 * float(b) * x ** 2 + 5 * float(c) * x ** 4
    np.testing.assert_allclose(deriv, 15 / 8 * (1 - x ** 2) ** 2, atol=1e-12)


def test_minimax_tends_to_limit_polynomial():
    diffs = []
    for d in (2e-2, 1e-2, 5e-3):
        coef = np.array(O.minimax_quintic(1 - d, 1 + d)[:3])
        diffs.append(np.max(np.abs(coef - np.array(O.LIMIT_QUINTIC))))
    # the best polynomial converges to the limit at rate d^2
    assert diffs[2] < diffs[1] < diffs[0] < 1e-2
    assert diffs[0] / diffs[1] == pytest.approx(4.0, rel=0.1)
    assert diffs[1] / diffs[2] == pytest.approx(4.0, rel=0.1)


def test_schedule_recursion():
    lo, margin = 1e-3, 0.02
    rows, E = O.minimax_schedule(6, lo, margin)
    l, u = lo, 1.0
    for k in range(6):
        a, b, c, Ek = O.minimax_quintic(l, u * (1 + margin))
        np.testing.assert_allclose(rows[k], [a, b, c], rtol=1e-12)
        l, u = 1 - Ek, 1 + Ek
    assert E == pytest.approx(Ek, rel=1e-12)


def test_schedule_without_margin_reaches_limit():
    rows, E = O.minimax_schedule(9, 1e-3, 0.0)
    assert tuple(rows[-1]) == O.LIMIT_QUINTIC
    assert E < 1e-15


@pytest.mark.parametrize("margin", [0.0, 0.02])
def test_schedule_bounds_every_value(margin):
    """Composed on a dense grid of [lo, 1], every value ends in [1-E, 1+E]."""
    lo = 1e-3
    x0 = np.concatenate([np.geomspace(lo, 1.0, 200001), np.linspace(lo, 1.0, 200001)])
    for T in range(1, 8):
        rows, E = O.minimax_schedule(T, lo, margin)
        x = x0.copy()
        for r in rows:
            x = O.quintic_eval(r, x)
        assert np.max(np.abs(1.0 - x)) <= E * (1 + 1e-9) + 1e-12


def test_schedule_beats_fixed_quintic():
    """Per-iteration coefficients: far smaller worst-case error for the same
    iteration count, and the fixed quintic never gets inside 0.3 of 1."""
    lo = 1e-3
    x0 = np.geomspace(lo, 1.0, 100001)
    fixed = (O.NS_A, O.NS_B, O.NS_C)
    x = x0.copy()
    for _ in range(5):
        x = O.quintic_eval(fixed, x)
    quintic_err5 = np.max(np.abs(1 - x))
    for _ in range(5):
        x = O.quintic_eval(fixed, x)
    quintic_err10 = np.max(np.abs(1 - x))
    # narrow margin: a third of the fixed quintic's error; default: 2.5x smaller
    assert O.minimax_schedule(5, lo, 0.02)[1] < quintic_err5 / 3
    assert O.minimax_schedule(5, lo)[1] < quintic_err5 / 2.5
    assert O.minimax_schedule(6, lo)[1] < 1e-2 < 0.3 < quintic_err10


def _svd_closed_form(Y, rows, eps=O.NS_EPS):
    Y = np.asarray(Y, dtype=np.float64)
    tall = Y.shape[0] > Y.shape[1]
    Z = Y.T if tall else Y
    U, s, Vt = np.linalg.svd(Z, full_matrices=False)
    s = s / (np.linalg.norm(Z) + eps)
    for r in rows:
        s = O.quintic_eval(r, s)
    X = (U * s) @ Vt
    return X.T if tall else X


@pytest.mark.parametrize("shape", [(24, 40), (40, 24), (32, 32)])
def test_ns_ref_rows_svd_closed_form(shape):
    rng = np.random.default_rng(shape[0] * 100 + shape[1])
    Y = rng.standard_normal(shape)
    rows, _ = O.minimax_schedule(5)
    got = O.ns_ref(Y, steps=5, coeffs=rows)
    ref = _svd_closed_form(Y, rows)
    np.testing.assert_allclose(got, ref, atol=1e-12 * np.abs(ref).max())
    # the order of the rows matters: reversed rows give another matrix
    rev = O.ns_ref(Y, steps=5, coeffs=rows[::-1])
    assert O.rel_fro(rev, ref) > 1e-2


def test_ns_ref_constant_rows_equal_fixed_coefficients():
    rng = np.random.default_rng(3)
    Y = rng.standard_normal((16, 48))
    rows = np.tile([O.NS_A, O.NS_B, O.NS_C], (4, 1))
    np.testing.assert_array_equal(O.ns_ref(Y, steps=4, coeffs=rows), O.ns_ref(Y, steps=4))


def test_ns_ref_rows_shape_checked():
    with pytest.raises(ValueError):
        O.ns_ref(np.ones((4, 8)), steps=3, coeffs=np.ones((2, 3)))


def test_schedule_argument_checks():
    for bad in [(0, 1e-3, 0.02), (3, 0.0, 0.02), (3, 1.0, 0.02), (3, 1e-3, -0.1), (3, 1e-3, 0.6)]:
        with pytest.raises(ValueError):
            O.minimax_schedule(*bad)
