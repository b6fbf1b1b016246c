"""Union and reuse of routing sets (test infrastructure only).

Lan, arXiv:2610.34440, Section 1 "Routing, union and reuse":
  X_t(n)  = |S_t u ... u S_{t+n-1}|, mean U(n), U(0) = 0;
  rho(n)  = (1/m) E|S_{t+n-1} n (S_t u ... u S_{t+n-2})|, rho(1) = 0   (Eq. 1);
  U(n)    = m sum_{j<=n} (1 - rho(j)) for every stationary process    (Eq. 2).
Appendix D.2 estimator: over every window of n consecutive tokens, count the last
token's experts that an earlier token of the window also selected; divide the sum
by m times the number of windows.
Section 3.4, Eq. (11): rho_bar_k = (1/(k W)) sum_{j=2..k+1} sum_l w_l rho_l(j).

A periodic pattern started at a uniformly random phase is stationary; its window
laws are the averages over the phases, computed here exactly with Fractions.
"""
from fractions import Fraction


def _sets(trace_ids):
    return [frozenset(int(e) for e in row) for row in trace_ids]


def union_windows(trace_ids, n):
    """X for every window [t, t+n) of a finite trace."""
    S = _sets(trace_ids)
    out = []
    for t in range(len(S) - n + 1):
        u = set()
        for s in S[t:t + n]:
            u |= s
        out.append(len(u))
    return out


def rho_hat(trace_ids, n, m):
    """Appendix D.2 window estimator of rho(n) on a finite trace (float)."""
    if n == 1:
        return 0.0
    S = _sets(trace_ids)
    hits = 0
    windows = 0
    for t in range(len(S) - n + 1):
        prev = set()
        for s in S[t:t + n - 1]:
            prev |= s
        hits += len(S[t + n - 1] & prev)
        windows += 1
    return hits / (m * windows)


def periodic_union(pattern, n):
    """Exact U(n) of a periodic pattern of expert sets at a uniform random phase."""
    S = _sets(pattern)
    P = len(S)
    tot = 0
    for ph in range(P):
        u = set()
        for i in range(n):
            u |= S[(ph + i) % P]
        tot += len(u)
    return Fraction(tot, P)


def periodic_rho(pattern, n, m):
    """Exact rho(n) (Eq. 1) of a periodic pattern at a uniform random phase."""
    if n == 1:
        return Fraction(0)
    S = _sets(pattern)
    P = len(S)
    tot = 0
    for ph in range(P):
        prev = set()
        for i in range(n - 1):
            prev |= S[(ph + i) % P]
        tot += len(S[(ph + n - 1) % P] & prev)
    return Fraction(tot, m * P)


def rho_bar(rhos_per_layer, w, k):
    """Eq. (11): rhos_per_layer[l][j] = rho_l(j) for j >= 1 (index j)."""
    W = sum(w)
    s = sum(w[l] * rhos_per_layer[l][j] for l in range(len(w)) for j in range(2, k + 2))
    return Fraction(s) / (k * W) if isinstance(s, Fraction) else s / (k * W)


def union_from_reuse(rhos, m, n):
    """Right side of Eq. (2): m sum_{j=1..n} (1 - rho(j)); rhos[j] = rho(j)."""
    return m * sum(1 - rhos[j] for j in range(1, n + 1))
