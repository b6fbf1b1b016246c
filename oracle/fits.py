"""Fits on passes with chosen ids, the bandwidth error and the error bounds.

TEST INFRASTRUCTURE ONLY.  Lan, arXiv:2610.34440:

* Section 2, Eq. (4): the per-slot kernel's time over passes whose nm slots name U
  distinct experts, t_slot = t_op + c_u U b + c_re (nm - U) b, fitted by least
  squares; c_re / c_u is the re-read cost.
* Appendix E, Eq. (E.1): the deduplicating kernel's time, t_dedup = t_op + c_g U b
  + c_t n, fitted the same way.
* Section 4, the prediction ahead of Section 4.1: epsilon_p is the median, over
  layers and models, of each fit's median relative error on the windows of
  recorded routing; an engine's epsilon is the larger of its two kernels' values.
* Section 3.5, Table 2, Appendix C: bounds for a relative bandwidth error
  |e| <= eps: (17) verify time, (18) saving, (19) faster kernel, and with a
  relative step-time error delta, (20) best draft length and (21) best speedup;
  from eps to delta: delta = eps / (1 - eps), so (1 + delta)/(1 - delta) =
  1/(1 - 2 eps).

The least-squares solve is numpy's (a library primitive); everything else is the
definition written out.
"""
import math

import numpy as np


def _lstsq(cols, t):
    A = np.column_stack([np.asarray(c, np.float64) for c in cols])
    coef, *_ = np.linalg.lstsq(A, np.asarray(t, np.float64), rcond=None)
    return tuple(float(c) for c in coef)


def fit_slot(n, U, m, t, b):
    """Eq. (4): (t_op, c_u, c_re) minimising sum (t - t_op - c_u U b - c_re (n m - U) b)^2."""
    n = np.asarray(n, np.float64)
    U = np.asarray(U, np.float64)
    return _lstsq([np.ones_like(U), U * b, (n * m - U) * b], t)


def fit_dedup(n, U, t, b):
    """Eq. (E.1): (t_op, c_g, c_t) minimising sum (t - t_op - c_g U b - c_t n)^2."""
    n = np.asarray(n, np.float64)
    U = np.asarray(U, np.float64)
    return _lstsq([np.ones_like(U), U * b, n], t)


def predict_slot(coef, n, U, m, b):
    t_op, c_u, c_re = coef
    return t_op + c_u * np.asarray(U, np.float64) * b + c_re * (np.asarray(n, np.float64) * m - U) * b


def predict_dedup(coef, n, U, b):
    t_op, c_g, c_t = coef
    return t_op + c_g * np.asarray(U, np.float64) * b + c_t * np.asarray(n, np.float64)


def median_rel_error(pred, meas):
    """A fit's median relative error |pred - meas| / meas over windows."""
    pred = np.asarray(pred, np.float64)
    meas = np.asarray(meas, np.float64)
    return float(np.median(np.abs(pred - meas) / meas))


def kernel_eps(median_errors):
    """epsilon_p: the median over layers (and models) of the fit's median relative errors."""
    return float(np.median(np.asarray(median_errors, np.float64)))


def engine_eps(eps_slot, eps_dedup):
    """An engine's epsilon: the larger of its two kernels' values."""
    return max(eps_slot, eps_dedup)


# ------------------------------ Table 2 ------------------------------

def verify_time_bound(eps, M):
    """(17): |tau^_p(n) - tau_p(n)| <= eps/(1 - eps) M_p(n) (<= eps/(1 - eps) tau_p(n))."""
    return eps / (1.0 - eps) * M


def saving_bound(eps, Me_slot, Me_dedup):
    """(18): |S^(n) - S(n)| <= eps/(1 - eps) (M^e_slot(n) + M^e_dedup(n))."""
    return eps / (1.0 - eps) * (Me_slot + Me_dedup)


def faster_kernel_agrees(r, u, eps):
    """(19): the two sides of (7) are decided alike by estimate and truth when
    |ln r(n) - ln u(n)| > ln((1 + eps)/(1 - eps))."""
    return abs(math.log(r) - math.log(u)) > math.log((1.0 + eps) / (1.0 - eps))


def delta_of_eps(eps):
    """From eps to delta (bandwidth errors alone, eps < 1/2): delta = eps/(1 - eps)."""
    return eps / (1.0 - eps)


def regret_factor(delta):
    """(20): T_a(k^*) >= (1 - delta)/(1 + delta) T_a(k*)."""
    return (1.0 - delta) / (1.0 + delta)


def kstar_separated(T, kstar, delta):
    """(20): k^* = k* when T_a(i) < (1 - delta)/(1 + delta) T_a(k*) for every i != k*."""
    f = regret_factor(delta)
    return all(T[i] < f * T[kstar] for i in range(len(T)) if i != kstar)


def speedup_interval(delta):
    """(21): (1 - delta)/(1 + delta) <= [T^_a(k^*)/T^_a(0)] / [T_a(k*)/T_a(0)] <= (1 + delta)/(1 - delta)."""
    return (1.0 - delta) / (1.0 + delta), (1.0 + delta) / (1.0 - delta)
