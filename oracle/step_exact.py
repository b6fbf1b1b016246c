"""Step-time model and best draft length in exact rational arithmetic.

TEST INFRASTRUCTURE ONLY.  Lan, arXiv:2610.34440:

* Section 1 "Speculative decoding": geometric acceptance, G_a(k) = 1 + a + ... + a^k,
  T_a(k) = G_a(k) / V(k), k*(a) = the smallest maximizer of T_a over 0..k_max,
  c_i = V(i) - V(i-1), step point a_j = inf{a in [0,1) : k*(a) >= j} (1 if none).
* Section 3.1, Eq. (5): tau_p(n) = t0 + D(n)/beta_D + E_p(n)/beta_p(n) + phi_p(n),
  D(n) = D + kv(n-1); V(k) = tau_p(k+1) + h(k); a one-token pass runs the same
  kernel either way (tau(1) carries no kernel index).  Eq. (6): the saving
  S(n) = tau_slot(n) - tau_dedup(n).
* Section 3.2, Eqs. (8)-(9) and Appendix B.1 (B.4): speedup condition, speedup,
  a0 = V(1)/V(0) - 1.
* Section 3.3 and Appendix B.3: alpha_{k,i} = inf{a : T_a(k) > T_a(i)} (1 if
  empty), a_j = max_{i<j} min_{k>=j} alpha_{k,i} (B.31); for convex
  non-decreasing V, a_1 = min(c_1/V(0), 1) (B.36).
* Section 3.4, Eqs. (14) and (16) (Appendix B.2, (B.14), (B.16)): reuse thresholds.
* Section 2: the crossover is the smallest pass size from which the saving
  stays positive.
"""
from fractions import Fraction as F


def G(a, k):
    return sum(F(a) ** i for i in range(k + 1))


def T(a, k, V):
    return G(a, k) / F(V[k])


def kstar(a, V):
    """Smallest maximizer of T_a(k) over k = 0..len(V)-1."""
    best = 0
    for k in range(1, len(V)):
        if T(a, k, V) > T(a, best, V):
            best = k
    return best


def a0(V):
    return F(V[1]) / F(V[0]) - 1


def faster(a, k, V):
    """Eq. (8): T_a(k) > T_a(0)  <=>  V(k) - V(0) < (a + ... + a^k) V(0)."""
    return F(V[k]) - F(V[0]) < (G(a, k) - 1) * F(V[0])


def speedup(a, k, V):
    """Eq. (9)."""
    return G(a, k) * F(V[0]) / F(V[k])


def _beats(a, k, i, V):
    return G(a, k) * F(V[i]) > G(a, i) * F(V[k])


def alpha_bracket(k, i, V, iters=60):
    """Bracket (lo, hi) of alpha_{k,i}: the predicate T_a(k) > T_a(i) is false
    below lo (or lo = 0) and true on (hi, 1) (Appendix B.3: the set is upward
    closed).  hi - lo <= 2^-iters unless the set is empty (then (1, 1)) or
    contains 0 (then (0, 0))."""
    if _beats(0, k, i, V):
        return F(0), F(0)
    # the set is upward closed in [0,1); empty iff the predicate fails just below 1
    lo, hi = F(0), F(1)
    near1 = 1 - F(1, 2 ** (iters + 8))
    if not _beats(near1, k, i, V):
        return F(1), F(1)
    for _ in range(iters):
        mid = (lo + hi) / 2
        if _beats(mid, k, i, V):
            hi = mid
        else:
            lo = mid
    return lo, hi


def step_point_bracket(j, V, iters=60):
    """(lo, hi) bracket of a_j = max_{i<j} min_{k>=j} alpha_{k,i} (B.31)."""
    K = len(V) - 1
    los, his = [], []
    for i in range(j):
        br = [alpha_bracket(k, i, V, iters) for k in range(j, K + 1)]
        los.append(min(b[0] for b in br))
        his.append(min(b[1] for b in br))
    return max(los), max(his)


def a1_convex(V):
    """(B.36): a_1 = min(c_1 / V(0), 1) when V is convex and non-decreasing."""
    return min((F(V[1]) - F(V[0])) / F(V[0]), F(1))


def is_convex_nondecreasing(V):
    c = [F(V[i]) - F(V[i - 1]) for i in range(1, len(V))]
    return all(x >= 0 for x in c) and all(c[i] <= c[i + 1] for i in range(len(c) - 1))


def tau(n, t0, D, kv, beta_D, E, beta, phi):
    """Eq. (5) for pass size n; kv[k] = kv(k), so D(n) = D + kv[n-1]."""
    return F(t0) + (F(D) + F(kv[n - 1])) / F(beta_D) + F(E) / F(beta) + F(phi)


def rho_star_time(k, a, m, W, tau1, beta1, Bk, dD, beta_D, dphi):
    """Eq. (14): 1 - (B_k/(mWk)) [(G_a(k)-1) tau(1) - dD/beta_D - dphi] - (B_k/beta(1) - 1)/k."""
    m, W, Bk, beta1 = F(m), F(W), F(Bk), F(beta1)
    bracket = (G(a, k) - 1) * F(tau1) - F(dD) / F(beta_D) - F(dphi)
    return 1 - Bk / (m * W * k) * bracket - (Bk / beta1 - 1) / k


def rho_star_bytes(k, a, m, W, D, kv):
    """Eq. (16): 1 - [(G_a(k)-1) V_dedup(0) - (kv(k) - kv(0))] / (m W k),
    V_dedup(0) = D + m W + kv(0)."""
    m, W = F(m), F(W)
    V0 = F(D) + m * W + F(kv[0])
    return 1 - ((G(a, k) - 1) * V0 - (F(kv[k]) - F(kv[0]))) / (m * W * k)


def crossover(S, n_max, n_min=2):
    """Smallest n in [n_min, n_max] with S(n') > 0 for every n' in [n, n_max];
    0 when there is none.  S maps n -> saving."""
    best = 0
    for n in range(n_max, n_min - 1, -1):
        if S[n] > 0:
            best = n
        else:
            break
    return best
