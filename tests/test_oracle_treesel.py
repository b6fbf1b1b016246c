"""Pins of the subtree-selection oracle (SpecFit, arXiv:2610.15417, Sections 3.1-3.3,
Appendix A.2/A.3): closed forms on hand-built pools, the equivalence of the ratio
rule with Eq. (6), nesting of Lemma 2, and the clique construction of Proposition 2."""
from fractions import Fraction as Fr
from itertools import combinations

from oracle import treesel as ts


def _pool_chain(V, E_root, E_nodes):
    parent = [-1] + [0] + list(range(1, V))
    return parent, [[set(E_root)]] + [[set(e)] for e in E_nodes]


def test_legal_family_counts_ancestor_closed_subsets():
    # root -> 1 -> {2, 3}: legal subsets of size <= 3: {}, {1}, {1,2}, {1,3}, {1,2,3}
    parent = [-1, 0, 1, 1]
    sets = [S for k in range(4) for S in combinations([1, 2, 3], k) if ts.legal(S, parent)]
    assert sets == [(), (1,), (1, 2), (1, 3), (1, 2, 3)]


def test_free_node_is_taken_and_costly_node_is_not():
    # node 1 brings no new expert: it raises R at no cost in F, and b is flat
    parent, E = [-1, 0, 0], [[{1, 2}], [{1}], [{7, 8, 9}]]
    p = [0, Fr(1, 2), Fr(1, 10)]
    S, R, F, T = ts.select(parent, p, E, 2, [10, 10, 10], 1)
    assert S == [1] and R == Fr(3, 2) and F == 2 and T == 12
    # with a large enough reward the costly node pays for itself: (1.5+1)/(10+5) > 1.5/12
    p[2] = Fr(1)
    assert ts.select(parent, p, E, 2, [10, 10, 10], 1)[0] == [1, 2]


def test_ratio_rule_matches_equation_6():
    # (R, T) beats (R0, T0) iff (T0 - T)/T0 > (R0 - R)/R0 (positive R, T)
    for R, T, R0, T0 in ((3, 10, 4, 14), (2, 5, 2, 6), (5, 9, 1, 2)):
        assert (Fr(R, T) > Fr(R0, T0)) == (Fr(T0 - T, T0) > Fr(R0 - R, R0))


def test_ties_prefer_reward_then_union_then_size_then_ids():
    parent, E = [-1, 0, 0], [[{0}], [{1}], [{2}]]
    p = [0, Fr(1), Fr(1)]
    # S={1} and S={2} tie on every key but the ids: the smaller id list wins
    S = ts.select(parent, p, E, 1, [1, 2], 1)[0]
    assert S == [1]


def test_adaptive_depth_nests_and_stops():
    parent = [-1, 0, 1, 2]
    level = [0, 1, 2, 3]
    E = [[{0}], [{0}], [{0}], [{5, 6, 7, 8}]]
    p = [0, Fr(9, 10), Fr(8, 10), Fr(1, 100)]
    b = [10, 10, 10, 10]
    sel, d = ts.select_adaptive(parent, p, E, 3, b, 1, level)
    assert sel == [1, 2] and d == 3  # level 3 adds only a costly node: the selection stops changing
    full = ts.select(parent, p, E, 3, b, 1)[0]
    assert full == sel  # Lemma 2: the stopped selection equals the full-pool selection here


def test_clique_construction_of_proposition_2():
    # one layer, one expert per vertex; a node per edge routes to its two vertices
    edges = [(0, 1), (1, 2), (0, 2), (2, 3)]  # a triangle 0-1-2 plus a pendant edge
    n_vert, r = 4, 3
    k, m_e = r * (r - 1) // 2, len(edges)
    p = Fr(1, m_e + 1)
    b = Fr(1)
    beta = b * p / (n_vert * (1 + (k - 1) * p)) / 2
    parent = [-1] + [0] * m_e
    E = [[set()]] + [[set(e)] for e in edges]
    S, R, F, T = ts.select(parent, [0] + [p] * m_e, E, k, [b] * (k + 1), beta)
    theta = (1 + k * p) / (b + beta * r)
    assert R / T >= theta and F == r and sorted(S) == [1, 2, 3]  # the triangle's edges
