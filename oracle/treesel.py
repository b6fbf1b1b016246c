"""Selection of the verification subtree by reward over predicted cycle time.

TEST INFRASTRUCTURE ONLY.  SpecFit (Cao et al., arXiv:2610.15417):

* Section 3.1, Eq. (2): the legal family A_K of ancestor-closed subsets S of the
  draft pool V (a node needs its parent in S or the root s) with |S| <= K.
* Section 3.2, Eq. (3): reward R(S) = 1 + sum_{v in S} p_v; Eq. (4): union feature
  F(S) = sum over layers l of |E_l(s) u U_{v in S} E_l(v)| and cycle time
  T(S) = b_|S| + beta F(S).
* Section 3.3, Eq. (5): the selection maximises R/T over A_K; equal ratios prefer the
  larger reward, the smaller union, fewer draft nodes, then the lexicographically
  smaller list of node ids.
* Appendix A.2, Lemma 2 (adaptive depth): the selection over the nodes of the first
  d levels; drafting stops at the first d whose selection equals that of d - 1.

Brute force over all subsets with exact rational arithmetic (inputs as Fractions or
numbers exactly representable as them); pools of up to ~16 nodes.
"""
from fractions import Fraction as Fr
from itertools import combinations


def legal(S, parent):
    s = set(S)
    return all(parent[v] == 0 or parent[v] in s for v in S)


def features(S, p, experts):
    """(R, F) of subset S; experts[v][l] = set of experts of node v (v = 0: root) in layer l."""
    R = 1 + sum(Fr(p[v]) for v in S)
    F = 0
    for l in range(len(experts[0])):
        u = set(experts[0][l])
        for v in S:
            u |= set(experts[v][l])
        F += len(u)
    return R, F


def select(parent, p, experts, K, b, beta, max_level=None, level=None):
    """The selected subset (sorted node ids), with its R, F, T."""
    V = len(parent) - 1
    nodes = [v for v in range(1, V + 1) if max_level is None or level[v] <= max_level]
    best = None
    for k in range(0, min(K, len(nodes)) + 1):
        for S in combinations(nodes, k):
            if not legal(S, parent):
                continue
            R, F = features(S, p, experts)
            T = Fr(b[len(S)]) + Fr(beta) * F
            key = (R / T, R, -F, -len(S))
            if best is None or key > best[0] or (key == best[0] and list(S) < best[1]):
                best = (key, list(S), R, F, T)
    return best[1], best[2], best[3], best[4]


def select_adaptive(parent, p, experts, K, b, beta, level):
    """Lemma 2: selections over the first d levels, d = 1, 2, ...; returns (selection
    at the stopping level, stopping level d, where the selection of d equals that of
    d - 1, or the deepest level)."""
    depth = max(level[1:])
    prev = select(parent, p, experts, K, b, beta, 0, level)[0]
    for d in range(1, depth + 1):
        cur = select(parent, p, experts, K, b, beta, d, level)[0]
        if cur == prev:
            return cur, d
        prev = cur
    return prev, depth
