"""The library's fits on chosen ids and Table 2 factors against the oracle (host
code, no GPU).  Lan, arXiv:2610.34440, Section 2 Eq. (4), Appendix E Eq. (E.1),
Section 3.5 Table 2."""
import math

import numpy as np
import pytest

import expert_ffn_amd as efa
from expert_ffn_amd import _abi
from oracle import fits


def _passes(rng, m, N, count):
    n = rng.integers(2, 10, size=count)
    U = np.array([rng.integers(m, min(a * m, N) + 1) for a in n])
    return n, U


@pytest.mark.parametrize("seed", range(6))
def test_fit_times_matches_oracle(seed):
    rng = np.random.default_rng(seed)
    m, N, b = 6, 64, 17_301_504
    n, U = _passes(rng, m, N, 40)
    t = 5e-6 + 1.9e-13 * U * b + 4e-14 * (n * m - U) * b
    t = t * (1 + 0.05 * rng.standard_normal(t.shape))
    got = efa.fit_times(efa.MOE_KIND_SLOT, n, U, m, t, b)
    assert np.allclose(got, fits.fit_slot(n, U, m, t, b), rtol=1e-9, atol=1e-20)
    t = 4e-6 + 2.2e-13 * U * b + 1.5e-6 * n
    t = t * (1 + 0.05 * rng.standard_normal(t.shape))
    got = efa.fit_times(efa.MOE_KIND_DEDUP, n, U, m, t, b)
    assert np.allclose(got, fits.fit_dedup(n, U, t, b), rtol=1e-9, atol=1e-20)


def test_fit_times_rejects_what_does_not_determine_the_fit():
    m, b = 4, 1000.0
    n = np.array([2, 3, 4, 5])
    with pytest.raises(_abi.MoeError):  # every slot distinct: c_re has nothing to fit
        efa.fit_times(efa.MOE_KIND_SLOT, n, n * m, m, np.ones(4), b)
    with pytest.raises(_abi.MoeError):  # fewer than three passes
        efa.fit_times(efa.MOE_KIND_DEDUP, n[:2], n[:2] * m, m, np.ones(2), b)
    with pytest.raises(_abi.MoeError):  # U above n m
        efa.fit_times(efa.MOE_KIND_DEDUP, n, n * m + 1, m, np.ones(4), b)


@pytest.mark.parametrize("eps", [0.0, 0.031, 0.054, 0.1, 0.148, 0.3, 0.49])
def test_error_bounds_match_oracle(eps):
    got = efa.error_bounds(eps)
    d = fits.delta_of_eps(eps)
    assert math.isclose(got["time_factor"], fits.verify_time_bound(eps, 1.0), rel_tol=1e-14, abs_tol=1e-15)
    assert math.isclose(got["delta"], d, rel_tol=1e-14, abs_tol=1e-15)
    assert math.isclose(got["regret_factor"], fits.regret_factor(d), rel_tol=1e-14)
    lo, hi = fits.speedup_interval(d)
    assert math.isclose(got["speedup_factor"], hi, rel_tol=1e-14) and math.isclose(1 / got["speedup_factor"], lo,
                                                                                     rel_tol=1e-12)
    # (19): the margin separates agreeing from undecided pairs exactly as the oracle does
    for lr in (0.5 * got["faster_margin"], 1.5 * got["faster_margin"] + 1e-9):
        assert (lr > got["faster_margin"]) == fits.faster_kernel_agrees(math.exp(lr), 1.0, eps)
    with pytest.raises(_abi.MoeError):
        efa.error_bounds(0.5)
