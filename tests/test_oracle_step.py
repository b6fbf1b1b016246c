"""Pins of the exact step-time oracle against what the pages print and prove.

* Appendix B.2 "No single threshold": rho*_1 = 7/20, rho*_2 = 371/800 by Eq. (16),
  speedup yes / yes / no for patterns 01, 00012, 00102.
* Appendix B.3 "Jumps": V = (1, 2, 2) gives k*(1/2) = 0, k*(9/10) = 2, never 1.
* Section 1: affine step time 1 + chi k: speculation wins exactly when a > chi.
* (B.4): one draft beats none exactly when a > a0 = V(1)/V(0) - 1.
* (B.28) monotone staircase; (B.31) step points; (10)/(B.35)-(B.36) for convex V,
  checked against brute-force argmax.
"""
import json
import os
import random
from fractions import Fraction as F

from oracle import step_exact as se

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_no_single_threshold_printed_values():
    g = json.load(open(os.path.join(GOLDEN, "no_single_threshold.json")))
    a = F(g["setup"]["a"])
    kv = [0, 0, 0]
    assert se.rho_star_bytes(1, a, 1, 1, 0, kv) == F(g["printed"]["rho_star"]["1"])
    assert se.rho_star_bytes(2, a, 1, 1, 0, kv) == F(g["printed"]["rho_star"]["2"])
    for row in g["printed"]["patterns"]:
        V = [F(v) for v in g["derived_not_printed"]["V"][row["pattern"]]]
        rb = {1: F(row["rho_bar_1"]), 2: F(row["rho_bar_2"])}
        rs = {k: se.rho_star_bytes(k, a, 1, 1, 0, kv) for k in (1, 2)}
        any_speed = any(rb[k] > rs[k] for k in (1, 2))
        assert any_speed == row["speedup"]
        # (B.14): the reuse form agrees with the time form (8) at every k
        for k in (1, 2):
            assert (rb[k] > rs[k]) == se.faster(a, k, V)
        if row["speedup_at_k"]:
            assert se.faster(a, row["speedup_at_k"], V)
        assert se.kstar(a, V) == g["derived_not_printed"]["kstar"][row["pattern"]]


def test_staircase_jump_printed():
    g = json.load(open(os.path.join(GOLDEN, "staircase_jump.json")))
    V = [F(v) for v in g["printed"]["V_dedup"]]
    for a, k in g["printed"]["kstar"].items():
        assert se.kstar(F(a), V) == k
    for i in range(0, 1000):
        assert se.kstar(F(i, 1000), V) != g["printed"]["kstar_never"]


def test_affine_step_time_threshold_is_chi():
    for chi in (F(1, 10), F(3, 7), F(9, 10)):
        V = [1 + chi * k for k in range(6)]
        lo, hi = se.step_point_bracket(1, V)
        assert lo <= chi <= hi and hi - lo < F(1, 2 ** 50)
        assert se.a1_convex(V) == chi
        assert se.kstar(chi - F(1, 10 ** 6), V) == 0 and se.kstar(chi + F(1, 10 ** 6), V) >= 1


def _rand_V(rng, K, convex=False):
    if convex:
        c = sorted(F(rng.randint(0, 40), 40) for _ in range(K))
        V = [F(1)]
        for ci in c:
            V.append(V[-1] + ci)
        return V
    return [F(rng.randint(20, 80), 40) for _ in range(K + 1)]


def test_a0_is_one_draft_threshold():
    rng = random.Random(3)
    for _ in range(50):
        V = _rand_V(rng, 3)
        a0 = se.a0(V)
        for a in (F(i, 37) for i in range(37)):
            assert (se.T(a, 1, V) > se.T(a, 0, V)) == (a > a0)
            assert se.faster(a, 1, V) == (a > a0)


def test_staircase_monotone_and_step_points():
    rng = random.Random(5)
    grid = [F(i, 97) for i in range(97)]
    for _ in range(40):
        V = _rand_V(rng, 4)
        ks = [se.kstar(a, V) for a in grid]
        assert all(ks[i] <= ks[i + 1] for i in range(len(ks) - 1))  # (B.28)
        for j in range(1, 5):
            lo, hi = se.step_point_bracket(j, V)
            for a in grid:
                if a > hi:
                    assert se.kstar(a, V) >= j
                if a < lo:
                    assert se.kstar(a, V) < j


def test_convex_step_condition_and_first_step_point():
    rng = random.Random(9)
    grid = [F(i, 61) for i in range(61)]
    for _ in range(40):
        V = _rand_V(rng, 5, convex=True)
        assert se.is_convex_nondecreasing(V)
        for a in grid:
            k = se.kstar(a, V)
            for j in range(1, 6):
                cj = V[j] - V[j - 1]
                assert (k >= j) == (a ** j * V[j - 1] > se.G(a, j - 1) * cj)  # Eq. (10)
        lo, hi = se.step_point_bracket(1, V)
        a1 = se.a1_convex(V)
        assert lo <= a1 <= hi or (a1 == 1 and hi == 1)


def test_time_threshold_reduces_to_byte_form():
    """(14) with one bandwidth and t0 = phi = 0 is (16) (Appendix B.2, 'One bandwidth')."""
    rng = random.Random(2)
    for _ in range(30):
        m, W, beta = rng.randint(1, 8), F(rng.randint(1, 50)), F(rng.randint(1, 9))
        D = F(rng.randint(0, 30))
        kv = [F(rng.randint(0, 5)) * i for i in range(6)]
        a = F(rng.randint(0, 99), 100)
        for k in range(1, 5):
            tau1 = (D + kv[0] + m * W) / beta
            t = se.rho_star_time(k, a, m, W, tau1, beta, beta, kv[k] - kv[0], beta, 0)
            assert t == se.rho_star_bytes(k, a, m, W, D, kv)


def test_crossover_definition():
    S = {2: -1, 3: -0.5, 4: 0.2, 5: 0.1, 6: 0.3}
    assert se.crossover(S, 6) == 4
    S = {2: 1, 3: -0.5, 4: 0.2}
    assert se.crossover(S, 4) == 4
    assert se.crossover({2: 1, 3: -1}, 3) == 0
