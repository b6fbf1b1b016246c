"""Pins of the oracle's union count and reuse estimators.

* Closed form under independent uniform routing (Lan, Section 1, citing MoESD):
  E[U(n)] = N (1 - q^n), q = 1 - m/N; exact over every pass of the tiny layer and
  statistically (4 sigma, exact variance) over many seeded passes of every shape.
* Reuse (Eq. 1), its estimator (Appendix D.2), the union identity (Eq. 2) and the
  byte-weighted mean reuse (Eq. 11) on the periodic patterns of Appendix B.2,
  whose rho_bar values the pages print.
"""
import itertools
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import reuse
from synth import routing

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_exact_enumeration_tiny_mean_union():
    N, m, n = 8, 2, 4
    sets = list(itertools.combinations(range(N), m))  # 28 unordered 2-subsets
    idx = np.array(list(itertools.product(range(len(sets)), repeat=n)), np.int32)  # 28^4 passes
    S = np.array(sets, np.int32)
    ids = S[idx]  # [B][n][m]
    U = oracle.union_count_batch(ids, N)
    q = Fraction(N - m, N)
    assert Fraction(int(U.sum()), ids.shape[0]) == N * (1 - q ** n) == Fraction(175, 32)


def _var_u(N, m, n):
    q = (N - m) / N
    q2 = (N - m) * (N - m - 1) / (N * (N - 1))
    return N * q ** n * (1 - q ** n) + N * (N - 1) * (q2 ** n - q ** (2 * n))


@pytest.mark.parametrize("N,m", [(8, 2), (64, 6), (128, 8)])
def test_closed_form_mean_union_over_seeds(N, m):
    S = 10000
    for n in (1, 2, 4, 8):
        tr = routing.uniform_trace(N, m, S * n, routing.rng_for(1234 + n, N, "uniform"))
        U = oracle.union_count_batch(tr.ids.reshape(S, n, m), N)
        q = 1 - m / N
        mean = N * (1 - q ** n)
        sd = np.sqrt(max(_var_u(N, m, n), 0.0))  # exactly 0 at n = 1
        assert abs(U.mean() - mean) <= 4 * sd / np.sqrt(S) + 1e-12, (n, U.mean(), mean)
        if n == 1:
            assert np.all(U == m)


def _pattern_sets(p):
    return [[int(c)] for c in p]


def test_periodic_patterns_printed_reuse():
    g = json.load(open(os.path.join(GOLDEN, "no_single_threshold.json")))
    for row in g["printed"]["patterns"]:
        pat = _pattern_sets(row["pattern"])
        rhos = {j: reuse.periodic_rho(pat, j, 1) for j in (1, 2, 3)}
        assert rhos[1] == 0
        rb1 = reuse.rho_bar([rhos], [1], 1)
        rb2 = reuse.rho_bar([rhos], [1], 2)
        assert rb1 == Fraction(row["rho_bar_1"]) and rb2 == Fraction(row["rho_bar_2"])
        # Eq. (2): U(n) = m sum_j (1 - rho(j)), exactly, on a stationary process
        for n in (1, 2, 3):
            assert reuse.periodic_union(pat, n) == reuse.union_from_reuse(rhos, 1, n)
        # the V of the derived table is U(k+1) with w = 1, D = kv = 0
        V = [reuse.periodic_union(pat, k + 1) for k in range(3)]
        assert V == [Fraction(v) for v in g["derived_not_printed"]["V"][row["pattern"]]]


def test_union_identity_on_random_cyclic_traces():
    rng = np.random.default_rng(7)
    for N, m, P in [(6, 2, 7), (10, 3, 11), (4, 1, 9)]:
        pat = [list(rng.choice(N, m, replace=False)) for _ in range(P)]
        rhos = {j: reuse.periodic_rho(pat, j, m) for j in range(1, 6)}
        for n in range(1, 6):
            assert reuse.periodic_union(pat, n) == reuse.union_from_reuse(rhos, m, n)


def test_uniform_reuse_closed_form_and_estimator():
    N, m, T = 64, 6, 40000
    tr = routing.uniform_trace(N, m, T, routing.rng_for(99, 0, "uniform"))
    q = 1 - m / N
    for n in (2, 3, 5):
        r = reuse.rho_hat(tr.ids, n, m)
        want = 1 - q ** (n - 1)
        assert abs(r - want) < 0.01, (n, r, want)
    # union windows agree with the C union count
    X = reuse.union_windows(tr.ids[:200], 4)
    U = [oracle.union_count(tr.ids[t:t + 4], N) for t in range(197)]
    assert X == U
