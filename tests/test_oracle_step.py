"""Pins of the exact step-time oracle against what the pages print and prove.

Every pin is a function ``pin_*(se)`` of the step-model module, so that the same
pins also run against planted mistakes in copies of it (test_oracle_step_mutants).

* Appendix B.2 "No single threshold": rho*_1 = 7/20, rho*_2 = 371/800 by Eq. (16),
  speedup yes / yes / no for patterns 01, 00012, 00102.
* Appendix B.3 "Jumps": V = (1, 2, 2) gives k*(1/2) = 0, k*(9/10) = 2, never 1.
* Section 1: affine step time 1 + chi k: speculation wins exactly when a > chi.
* (B.4): one draft beats none exactly when a > a0 = V(1)/V(0) - 1.
* (B.28) monotone staircase; (B.31) step points; (10)/(B.35)-(B.36) for convex V,
  checked against brute-force argmax.
* Section 1 "Speculative decoding" with Appendix B.2 "One bandwidth": a step that
  drafts k tokens requests D + E_p(k+1) + kv(k) bytes, and with one bandwidth and
  t0 = phi = 0 the step time (5) is that byte count over the bandwidth.  This pins
  the KV index of Eq. (5) (D(n) = D + kv(n-1)) by a statement other than (5).
* Eq. (13) (a draft's added time, term by term), Eq. (9) against the throughput
  ratio T_a(k)/T_a(0) taken from its definition, Eq. (15), and (B.14): on random
  models with two bandwidths (B_k != beta(1)), fixed work that differs between
  pass sizes and non-linear KV bytes, rho_bar_k > rho*_k(a) exactly when
  T_a(k) > T_a(0), with E_dedup(k+1) = mW + mWk(1 - rho_bar_k) (Eq. 12).  Every term
  of the time-form threshold (14) moves the decision on some of these models.
* (B.18) the explicit one-draft forms of rho*_1 and a0; (B.19) how the threshold
  moves with a and with D; (B.22) the one-bandwidth a0.
"""
import json
import os
import random
from fractions import Fraction as F

from oracle import step_exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _geo(a, k):
    """Expected tokens of a step drafting k under geometric acceptance (Section 1), summed here."""
    return sum(F(a) ** i for i in range(k + 1))


def pin_no_single_threshold_printed_values(se):
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


def pin_staircase_jump_printed(se):
    g = json.load(open(os.path.join(GOLDEN, "staircase_jump.json")))
    V = [F(v) for v in g["printed"]["V_dedup"]]
    for a, k in g["printed"]["kstar"].items():
        assert se.kstar(F(a), V) == k
    for i in range(0, 1000):
        assert se.kstar(F(i, 1000), V) != g["printed"]["kstar_never"]


def pin_affine_step_time_threshold_is_chi(se):
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


def pin_a0_is_one_draft_threshold(se):
    rng = random.Random(3)
    for _ in range(50):
        V = _rand_V(rng, 3)
        a0 = se.a0(V)
        for a in (F(i, 37) for i in range(37)):
            assert (_geo(a, 1) / V[1] > _geo(a, 0) / V[0]) == (a > a0)
            assert (se.T(a, 1, V) > se.T(a, 0, V)) == (a > a0)
            assert se.faster(a, 1, V) == (a > a0)


def pin_staircase_monotone_and_step_points(se):
    rng = random.Random(5)
    grid = [F(i, 97) for i in range(97)]
    for _ in range(40):
        V = _rand_V(rng, 4)
        ks = [se.kstar(a, V) for a in grid]
        # the smallest maximizer of T_a(k) = G_a(k)/V(k) by brute force (Section 1)
        for a, k in zip(grid, ks):
            T = [_geo(a, j) / V[j] for j in range(len(V))]
            assert k == T.index(max(T))
        assert all(ks[i] <= ks[i + 1] for i in range(len(ks) - 1))  # (B.28)
        for j in range(1, 5):
            lo, hi = se.step_point_bracket(j, V)
            for a in grid:
                if a > hi:
                    assert se.kstar(a, V) >= j
                if a < lo:
                    assert se.kstar(a, V) < j


def pin_convex_step_condition_and_first_step_point(se):
    rng = random.Random(9)
    grid = [F(i, 61) for i in range(61)]
    for _ in range(40):
        V = _rand_V(rng, 5, convex=True)
        assert se.is_convex_nondecreasing(V)
        for a in grid:
            k = se.kstar(a, V)
            for j in range(1, 6):
                cj = V[j] - V[j - 1]
                assert (k >= j) == (a ** j * V[j - 1] > _geo(a, j - 1) * cj)  # Eq. (10)
        lo, hi = se.step_point_bracket(1, V)
        a1 = se.a1_convex(V)
        assert lo <= a1 <= hi or (a1 == 1 and hi == 1)


def pin_time_threshold_reduces_to_byte_form(se):
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


def pin_crossover_definition(se):
    S = {2: -1, 3: -0.5, 4: 0.2, 5: 0.1, 6: 0.3}
    assert se.crossover(S, 6) == 4
    S = {2: 1, 3: -0.5, 4: 0.2}
    assert se.crossover(S, 4) == 4
    assert se.crossover({2: 1, 3: -1}, 3) == 0
    # a saving of exactly zero is not a positive saving (Section 2: the first n from
    # which the saving stays positive)
    assert se.crossover({2: 0, 3: 1, 4: 2}, 4) == 3
    assert se.crossover({2: 1, 3: 0}, 3) == 0


def _kv_nonlinear(rng, K):
    """KV bytes kv(0..K+1), kv(0) >= 0 and increasing by unequal steps (so that an
    index off by one changes every difference)."""
    kv = [F(rng.randint(0, 4))]
    for _ in range(K + 1):
        kv.append(kv[-1] + F(rng.randint(1, 9), rng.randint(1, 3)) + F(len(kv) ** 2, 3))
    return kv


def pin_step_bytes_one_bandwidth(se):
    """Section 1: a step that drafts k tokens requests D + E_p(k+1) + kv(k) bytes; with
    one bandwidth beta for every byte and t0 = phi = 0 (Appendix B.2 'One bandwidth')
    its time (5) is those bytes over beta, so a plain step (k = 0) reads kv(0) and no
    later KV bytes."""
    rng = random.Random(21)
    for _ in range(60):
        K = rng.randint(1, 6)
        kv = _kv_nonlinear(rng, K)
        D = F(rng.randint(0, 40))
        beta = F(rng.randint(1, 13), rng.randint(1, 5))
        for k in range(0, K + 1):
            E = F(rng.randint(1, 100))
            assert se.tau(k + 1, 0, D, kv, beta, E, beta, 0) == (D + E + kv[k]) / beta
        # a plain step does not depend on the KV bytes of draft positions
        kv2 = kv[:1] + [v + 1000 for v in kv[1:]]
        assert se.tau(1, 0, D, kv, beta, F(7), beta, 0) == se.tau(1, 0, D, kv2, beta, F(7), beta, 0)
        # Section 3.1: t0 is time outside the memory reads, so a pass that reads nothing
        # and has no fixed work takes t0, and t0 adds to every pass one for one
        t0 = F(rng.randint(1, 30), 7)
        assert se.tau(rng.randint(1, K + 1), t0, 0, [0] * (K + 2), beta, 0, beta, 0) == t0
        n = rng.randint(1, K + 1)
        assert se.tau(n, t0, D, kv, beta, F(5), beta, F(1, 3)) - se.tau(n, 0, D, kv, beta, F(5), beta, F(1, 3)) == t0


def _two_bandwidth_model(rng, K):
    """A deduplicating engine with h = 0 (Appendix B.2 'Step time (13)'): per-slot
    one-token pass (beta(1), phi(1)), deduplicating passes with their own B_k and
    phi_dedup(k+1), non-linear KV, t0 > 0, D > 0, several experts per token."""
    M = dict(m=rng.randint(1, 8), W=F(rng.randint(5, 60)), t0=F(rng.randint(0, 9), 4), D=F(rng.randint(1, 90)),
             beta_D=F(rng.randint(2, 20), rng.randint(1, 3)), kv=_kv_nonlinear(rng, K))
    M["beta1"] = F(rng.randint(3, 30), rng.randint(1, 4))
    M["phi1"] = F(rng.randint(0, 20), 10)
    M["B"] = [None] + [M["beta1"] * F(rng.randint(40, 160), 100) for _ in range(K)]   # B_k != beta(1) in general
    M["phid"] = [None] + [M["phi1"] + F(rng.randint(-10, 30), 10) for _ in range(K)]
    M["phid"] = [None] + [max(p, F(0)) for p in M["phid"][1:]]
    return M


def _V(se, M, k, rho_bar):
    """V(0) = tau(1) (a one-token pass, no kernel index); V(k) = tau_dedup(k+1) with the
    union bytes of Eq. (12)."""
    mW = M["m"] * M["W"]
    if k == 0:
        return se.tau(1, M["t0"], M["D"], M["kv"], M["beta_D"], mW, M["beta1"], M["phi1"])
    E = mW + mW * k * (1 - rho_bar)
    return se.tau(k + 1, M["t0"], M["D"], M["kv"], M["beta_D"], E, M["B"][k], M["phid"][k])


def pin_time_threshold_decides_speedup(se):
    """(13), (9), (15) and (B.14) on random two-bandwidth models."""
    rng = random.Random(13)
    checked = decided_by_phi = decided_by_bk = 0
    for _ in range(80):
        K = rng.randint(1, 5)
        M = _two_bandwidth_model(rng, K)
        mW = M["m"] * M["W"]
        for k in range(1, K + 1):
            dD = M["kv"][k] - M["kv"][0]          # D(k+1) - D(1)
            dphi = M["phid"][k] - M["phi1"]
            for _ in range(4):
                rho = F(rng.randint(0, 100), 100)
                a = F(rng.randint(0, 99), 100)
                V0, Vk = _V(se, M, 0, rho), _V(se, M, k, rho)
                E = mW + mW * k * (1 - rho)
                # (13): the time a draft of length k adds
                assert Vk - V0 == E / M["B"][k] - mW / M["beta1"] + dD / M["beta_D"] + dphi
                # (9) against the throughput ratio, and (15)
                ratio = (_geo(a, k) / Vk) / (_geo(a, 0) / V0)
                V = [V0] + [None] * (k - 1) + [Vk]
                assert se.speedup(a, k, V) == ratio
                assert ratio == _geo(a, k) * V0 / (V0 + dD / M["beta_D"] + dphi + E / M["B"][k] - mW / M["beta1"])
                # (B.14): reuse above the threshold exactly when k drafts beat none
                rs = se.rho_star_time(k, a, M["m"], M["W"], V0, M["beta1"], M["B"][k], dD, M["beta_D"], dphi)
                faster = _geo(a, k) / Vk > _geo(a, 0) / V0
                assert (rho > rs) == faster
                checked += 1
                # the same decision with the fixed-work difference or the bandwidth ratio
                # dropped would differ on some of these models
                rs_nophi = se.rho_star_time(k, a, M["m"], M["W"], V0, M["beta1"], M["B"][k], dD, M["beta_D"], 0)
                decided_by_phi += (rho > rs_nophi) != faster
                rs_onebw = se.rho_star_time(k, a, M["m"], M["W"], V0, M["B"][k], M["B"][k], dD, M["beta_D"], dphi)
                decided_by_bk += (rho > rs_onebw) != faster
    assert checked > 500 and decided_by_phi > 0 and decided_by_bk > 0


def pin_one_draft_explicit_forms(se):
    """(B.18): rho*_1(a) = 1 - (B_1/(mW)) [a tau(1) - dD_1/beta_D - dphi_1] - (B_1/beta(1) - 1)
    and a0 = [dD_1/beta_D + dphi_1 + mW(2 - rho_bar_1)/B_1 - mW/beta(1)] / tau(1); one
    draft beats none exactly when rho_bar_1 > rho*_1(a), equivalently a > a0."""
    rng = random.Random(17)
    for _ in range(60):
        M = _two_bandwidth_model(rng, 1)
        mW = M["m"] * M["W"]
        dD, dphi, B1 = M["kv"][1] - M["kv"][0], M["phid"][1] - M["phi1"], M["B"][1]
        rho = F(rng.randint(0, 100), 100)
        V0, V1 = _V(se, M, 0, rho), _V(se, M, 1, rho)
        a0 = (dD / M["beta_D"] + dphi + mW * (2 - rho) / B1 - mW / M["beta1"]) / V0
        assert se.a0([V0, V1]) == a0
        for a in (F(i, 23) for i in range(23)):
            want = 1 - (B1 / mW) * (a * V0 - dD / M["beta_D"] - dphi) - (B1 / M["beta1"] - 1)
            rs = se.rho_star_time(1, a, M["m"], M["W"], V0, M["beta1"], B1, dD, M["beta_D"], dphi)
            assert rs == want
            assert (rho > rs) == (a > a0)


def pin_threshold_movement(se):
    """(B.19): moving a changes rho*_k by B_k tau(1)/(mWk) (G_a'(k) - G_a(k)); moving D to
    D' changes tau(1) by (D' - D)/beta_D and rho*_k by B_k (G_a(k) - 1)/(mWk) (D' - D)/beta_D;
    the threshold falls strictly as a grows."""
    rng = random.Random(19)
    for _ in range(40):
        K = rng.randint(1, 4)
        M = _two_bandwidth_model(rng, K)
        mW = M["m"] * M["W"]
        tau1 = _V(se, M, 0, 0)
        M2 = dict(M, D=M["D"] + F(rng.randint(1, 50)))
        tau1b = _V(se, M2, 0, 0)
        assert tau1b - tau1 == (M2["D"] - M["D"]) / M["beta_D"]
        for k in range(1, K + 1):
            dD, dphi, Bk = M["kv"][k] - M["kv"][0], M["phid"][k] - M["phi1"], M["B"][k]
            a, a2 = sorted(F(rng.randint(0, 99), 100) for _ in range(2))
            r = lambda aa, t1: se.rho_star_time(k, aa, M["m"], M["W"], t1, M["beta1"], Bk, dD, M["beta_D"], dphi)  # noqa
            assert r(a, tau1) - r(a2, tau1) == Bk * tau1 / (mW * k) * (_geo(a2, k) - _geo(a, k))
            if a2 > a:
                assert r(a2, tau1) < r(a, tau1)
            assert r(a, tau1) - r(a, tau1b) == Bk * (_geo(a, k) - 1) / (mW * k) * (M2["D"] - M["D"]) / M["beta_D"]


def pin_one_bandwidth_a0(se):
    """(B.22): with one bandwidth and t0 = phi = 0, a0 = [mW(1 - rho_bar_1) + kv(1) - kv(0)] / V_dedup(0),
    V_dedup(0) = D + mW + kv(0) (the byte count of a plain step)."""
    rng = random.Random(23)
    for _ in range(60):
        m, W = rng.randint(1, 8), F(rng.randint(1, 40))
        mW = m * W
        D, beta = F(rng.randint(0, 50)), F(rng.randint(1, 9), rng.randint(1, 4))
        kv = _kv_nonlinear(rng, 2)
        rho = F(rng.randint(0, 100), 100)
        V0 = se.tau(1, 0, D, kv, beta, mW, beta, 0)
        V1 = se.tau(2, 0, D, kv, beta, mW * (2 - rho), beta, 0)
        assert se.a0([V0, V1]) == (mW * (1 - rho) + kv[1] - kv[0]) / (D + mW + kv[0])


PINS = [pin_no_single_threshold_printed_values, pin_staircase_jump_printed, pin_affine_step_time_threshold_is_chi,
        pin_a0_is_one_draft_threshold, pin_staircase_monotone_and_step_points,
        pin_convex_step_condition_and_first_step_point, pin_time_threshold_reduces_to_byte_form,
        pin_crossover_definition, pin_step_bytes_one_bandwidth, pin_time_threshold_decides_speedup,
        pin_one_draft_explicit_forms, pin_threshold_movement, pin_one_bandwidth_a0]


def test_no_single_threshold_printed_values():
    pin_no_single_threshold_printed_values(step_exact)


def test_staircase_jump_printed():
    pin_staircase_jump_printed(step_exact)


def test_affine_step_time_threshold_is_chi():
    pin_affine_step_time_threshold_is_chi(step_exact)


def test_a0_is_one_draft_threshold():
    pin_a0_is_one_draft_threshold(step_exact)


def test_staircase_monotone_and_step_points():
    pin_staircase_monotone_and_step_points(step_exact)


def test_convex_step_condition_and_first_step_point():
    pin_convex_step_condition_and_first_step_point(step_exact)


def test_time_threshold_reduces_to_byte_form():
    pin_time_threshold_reduces_to_byte_form(step_exact)


def test_crossover_definition():
    pin_crossover_definition(step_exact)


def test_step_bytes_one_bandwidth():
    pin_step_bytes_one_bandwidth(step_exact)


def test_time_threshold_decides_speedup():
    pin_time_threshold_decides_speedup(step_exact)


def test_one_draft_explicit_forms():
    pin_one_draft_explicit_forms(step_exact)


def test_threshold_movement():
    pin_threshold_movement(step_exact)


def test_one_bandwidth_a0():
    pin_one_bandwidth_a0(step_exact)
