"""Planted mistakes in copies of the exact step-time oracle must each fail a pin.

Each mutant is ``oracle/step_exact.py`` with one plausible slip (an index off by one,
a flipped sign, an inverted ratio, a dropped term, the largest maximizer taken for
the smallest), loaded as a separate module; the pins of test_oracle_step run against
it and at least one must fail.  This shows that the step-model pins constrain every
part of it: Eq. (5) (its KV index and fixed work), Eq. (8), (9), (14) (each term),
(16), (B.4), (B.36), G_a(k) and the crossover rule.
"""
import types

import pytest

from oracle import step_exact

from . import test_oracle_step as T

MUTANTS = {
    "tau_kv_index": ("F(kv[n - 1])", "F(kv[n])"),
    "tau_phi_dropped": (" + F(E) / F(beta) + F(phi)", " + F(E) / F(beta)"),
    "tau_t0_dropped": ("return F(t0) + (F(D)", "return (F(D)"),
    "rho_time_dphi_sign": ("- F(dD) / F(beta_D) - F(dphi)", "- F(dD) / F(beta_D) + F(dphi)"),
    "rho_time_dD_sign": ("- F(dD) / F(beta_D) - F(dphi)", "+ F(dD) / F(beta_D) - F(dphi)"),
    "rho_time_bk_inverted": ("(Bk / beta1 - 1) / k", "(beta1 / Bk - 1) / k"),
    "rho_time_ratio_term_dropped": ("bracket - (Bk / beta1 - 1) / k", "bracket"),
    "rho_time_G_not_minus_one": ("bracket = (G(a, k) - 1) * F(tau1)", "bracket = G(a, k) * F(tau1)"),
    "speedup_inverted": ("return G(a, k) * F(V[0]) / F(V[k])", "return G(a, k) * F(V[k]) / F(V[0])"),
    "speedup_G_minus_one": ("return G(a, k) * F(V[0]) / F(V[k])", "return (G(a, k) - 1) * F(V[0]) / F(V[k])"),
    "kstar_largest_maximizer": ("if T(a, k, V) > T(a, best, V):", "if T(a, k, V) >= T(a, best, V):"),
    "a0_minus_one_dropped": ("return F(V[1]) / F(V[0]) - 1", "return F(V[1]) / F(V[0])"),
    "faster_G_not_minus_one": ("< (G(a, k) - 1) * F(V[0])", "< G(a, k) * F(V[0])"),
    "rho_bytes_kv_sign": ("- (F(kv[k]) - F(kv[0]))", "+ (F(kv[k]) - F(kv[0]))"),
    "rho_bytes_V0_without_D": ("V0 = F(D) + m * W + F(kv[0])", "V0 = m * W + F(kv[0])"),
    "G_one_term_short": ("for i in range(k + 1))", "for i in range(k))"),
    "a1_over_V1": ("min((F(V[1]) - F(V[0])) / F(V[0]), F(1))", "min((F(V[1]) - F(V[0])) / F(V[1]), F(1))"),
    "crossover_zero_counts": ("        if S[n] > 0:", "        if S[n] >= 0:"),
}


def _mutant_module(name):
    old, new = MUTANTS[name]
    src = open(step_exact.__file__).read()
    assert src.count(old) == 1, "mutation site of %s not unique in the step oracle" % name
    mod = types.ModuleType("step_exact_" + name)
    mod.__file__ = step_exact.__file__
    exec(compile(src.replace(old, new), "<mutant %s>" % name, "exec"), mod.__dict__)
    return mod


def _run_pins(mod, stop_at_first=False):
    """Names of the pins that fail on `mod`, cheapest pins first."""
    failed = []
    for pin in sorted(T.PINS, key=lambda p: p in SLOW_PINS):
        try:
            pin(mod)
        except (AssertionError, ZeroDivisionError, IndexError, TypeError):
            failed.append(pin.__name__)
            if stop_at_first:
                break
    return failed


SLOW_PINS = (T.pin_staircase_monotone_and_step_points, T.pin_convex_step_condition_and_first_step_point)


def test_unmutated_copy_passes_every_pin():
    src = open(step_exact.__file__).read()
    mod = types.ModuleType("step_exact_copy")
    exec(compile(src, "<copy>", "exec"), mod.__dict__)
    assert _run_pins(mod) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_step_mistake_is_caught(name):
    failed = _run_pins(_mutant_module(name), stop_at_first=True)
    assert failed, "no pin caught the planted mistake %s" % name
