"""Pins of the fits on chosen ids (Eqs. (4), (E.1)) and the Table 2 bounds.

Lan, arXiv:2610.34440, Section 2 (fits), Section 3.5 / Table 2 / Appendix C
(bounds), Section 4 (epsilon).  The fits are pinned to the exact least-squares
solution of small integer systems (normal equations in rationals); the bounds
to the step-time model of Eq. (5) under bandwidth errors drawn within eps, to
their tightness at e = -eps, and to the printed factor 1.25 at eps = 0.1.
"""
import math
import random
from fractions import Fraction as F

import numpy as np

from oracle import fits
from oracle import step_exact as se


def _exact_lstsq(cols, t):
    """Least squares by the normal equations in exact rationals (Gauss-Jordan)."""
    k = len(cols)
    A = [[sum(F(cols[i][r]) * F(cols[j][r]) for r in range(len(t))) for j in range(k)] for i in range(k)]
    y = [sum(F(cols[i][r]) * F(t[r]) for r in range(len(t))) for i in range(k)]
    for c in range(k):
        p = next(r for r in range(c, k) if A[r][c] != 0)
        A[c], A[p] = A[p], A[c]
        y[c], y[p] = y[p], y[c]
        for r in range(k):
            if r != c and A[r][c] != 0:
                f = A[r][c] / A[c][c]
                A[r] = [a - f * b for a, b in zip(A[r], A[c])]
                y[r] -= f * y[c]
    return [y[i] / A[i][i] for i in range(k)]


def test_fits_equal_exact_least_squares():
    rng = random.Random(5)
    for trial in range(20):
        m, b = rng.randint(1, 8), rng.randint(1, 50)
        rows = []
        for _ in range(rng.randint(4, 12)):
            n = rng.randint(2, 9)
            U = rng.randint(m, n * m)
            rows.append((n, U, rng.randint(1, 1000)))
        n, U, t = (list(v) for v in zip(*rows))
        ex = _exact_lstsq([[1] * len(n), [u * b for u in U], [(a * m - u) * b for a, u in zip(n, U)]], t)
        got = fits.fit_slot(n, U, m, t, b)
        # rank-deficient draws (U = n m everywhere, ...) have no unique solution: skip
        if np.linalg.matrix_rank(np.column_stack([np.ones(len(n)), np.array(U) * b,
                                                  (np.array(n) * m - np.array(U)) * b])) == 3:
            assert np.allclose(got, [float(v) for v in ex], rtol=1e-9, atol=1e-9), (trial, got, ex)
        ex = _exact_lstsq([[1] * len(n), [u * b for u in U], n], t)
        got = fits.fit_dedup(n, U, t, b)
        if np.linalg.matrix_rank(np.column_stack([np.ones(len(n)), np.array(U) * b, np.array(n)])) == 3:
            assert np.allclose(got, [float(v) for v in ex], rtol=1e-9, atol=1e-9), (trial, got, ex)


def test_fits_recover_noiseless_coefficients():
    b, m = 17_301_504, 6
    n = [2, 2, 3, 3, 5, 8, 8, 9]
    U = [6, 12, 7, 18, 20, 6, 48, 30]
    t = [4e-6 + 2e-13 * u * b + 5e-14 * (a * m - u) * b for a, u in zip(n, U)]
    assert np.allclose(fits.fit_slot(n, U, m, t, b), (4e-6, 2e-13, 5e-14), rtol=1e-8)
    t = [3e-6 + 2.5e-13 * u * b + 1e-6 * a for a, u in zip(n, U)]
    assert np.allclose(fits.fit_dedup(n, U, t, b), (3e-6, 2.5e-13, 1e-6), rtol=1e-8)


def test_eps_is_median_then_larger_kernel():
    assert math.isclose(fits.median_rel_error([1.1, 0.8, 1.0], [1.0, 1.0, 1.0]), 0.1)
    assert math.isclose(fits.median_rel_error([3.0, 2.0], [2.0, 4.0]), 0.5)  # (0.5 + 0.5) / 2
    assert fits.kernel_eps([0.05, 0.02, 0.03]) == 0.03
    assert fits.engine_eps(0.031, 0.054) == 0.054


def test_printed_factor_at_ten_percent():
    # Section 3.5: a 10 % bandwidth error moves the predicted speedup by at most 25 %
    d = F(1, 10) / (1 - F(1, 10))
    assert (1 + d) / (1 - d) == F(5, 4) == 1 / (1 - 2 * F(1, 10))
    lo, hi = fits.speedup_interval(fits.delta_of_eps(0.1))
    assert math.isclose(hi, 1.25) and math.isclose(lo, 0.8)


def _tau(E_D, beta_D, E, beta, t0=0.0, phi=0.0):
    """Eq. (5) with one memory term each for the dense and the expert bytes."""
    return t0 + E_D / beta_D + E / beta + phi


def test_verify_and_saving_bounds_hold_and_are_tight():
    rng = random.Random(11)
    for _ in range(400):
        eps = rng.uniform(0.0, 0.45)
        D, bD = rng.uniform(0, 5e7), rng.uniform(1e11, 6e12)
        Es, bs = rng.uniform(1e7, 9e8), rng.uniform(1e11, 6e12)
        Ed, bd = rng.uniform(1e7, 9e8), rng.uniform(1e11, 6e12)
        t0, phi = rng.uniform(0, 1e-5), rng.uniform(0, 1e-5)
        eD, es, ed = (rng.uniform(-eps, eps) for _ in range(3))
        ts, td = _tau(D, bD, Es, bs, t0, phi), _tau(D, bD, Ed, bd, t0, phi)
        ts_h = _tau(D, bD * (1 + eD), Es, bs * (1 + es), t0, phi)
        td_h = _tau(D, bD * (1 + eD), Ed, bd * (1 + ed), t0, phi)
        Ms = D / bD + Es / bs
        assert abs(ts_h - ts) <= fits.verify_time_bound(eps, Ms) * (1 + 1e-12) + 1e-18
        assert fits.verify_time_bound(eps, Ms) <= fits.verify_time_bound(eps, ts) + 1e-18
        S, S_h = ts - td, ts_h - td_h
        assert abs(S_h - S) <= fits.saving_bound(eps, Es / bs, Ed / bd) * (1 + 1e-12) + 1e-18
        # tight: every bandwidth under-estimated by eps moves M by exactly the bound
        Ms_w = D / (bD * (1 - eps)) + Es / (bs * (1 - eps))
        assert math.isclose(Ms_w - Ms, fits.verify_time_bound(eps, Ms), rel_tol=1e-9, abs_tol=1e-18)


def test_faster_kernel_decision_agrees_beyond_margin_and_can_flip_inside():
    rng = random.Random(3)
    for _ in range(500):
        eps = rng.uniform(0.01, 0.4)
        x, y = rng.uniform(1e-6, 1e-3), rng.uniform(1e-6, 1e-3)   # true expert times
        phi = rng.uniform(0, 1e-4)                                 # equal fixed work
        r_over_u = y / x                                           # x / y = u / r
        agrees = fits.faster_kernel_agrees(r_over_u, 1.0, eps)
        for _ in range(20):
            u_, v_ = 1 / (1 + rng.uniform(-eps, eps)), 1 / (1 + rng.uniform(-eps, eps))
            if agrees:
                assert ((x * u_ + phi) < (y * v_ + phi)) == ((x + phi) < (y + phi))
        if not agrees and x != y:
            # inside the margin some errors within eps reverse the predicted order
            lo, hi = 1 / (1 + eps), 1 / (1 - eps)
            flip = (x * hi > y * lo) if x < y else (x * lo < y * hi)
            assert flip


def test_best_draft_length_and_speedup_bounds():
    rng = random.Random(7)
    for _ in range(300):
        K = rng.randint(1, 7)
        V = [F(rng.randint(100, 400))]
        for _k in range(K):
            V.append(V[-1] + F(rng.randint(1, 120)))
        a = F(rng.randint(0, 99), 100)
        delta = rng.uniform(0.0, 0.3)
        Vh = [v * F(1 + rng.uniform(-delta, delta)) for v in V]
        k, kh = se.kstar(a, V), se.kstar(a, Vh)
        T = [se.T(a, i, V) for i in range(K + 1)]
        assert float(T[kh]) >= fits.regret_factor(delta) * float(T[k]) * (1 - 1e-12)
        if fits.kstar_separated([float(v) for v in T], k, delta):
            assert kh == k
        lo, hi = fits.speedup_interval(delta)
        ratio = float((se.T(a, kh, Vh) / se.T(a, 0, Vh)) / (T[k] / T[0]))
        assert lo * (1 - 1e-12) <= ratio <= hi * (1 + 1e-12)
