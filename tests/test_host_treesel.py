"""The library's subtree selection (moe_tree_select) against the brute-force oracle
(SpecFit, arXiv:2610.15417, Sections 3.1-3.3, Algorithm 1, Appendix A.2).  Inputs are
multiples of 1/8 so that every double the search forms is exact and both sides take
the same decisions."""
from fractions import Fraction as Fr
from functools import lru_cache

import numpy as np
import pytest

import expert_ffn_amd as efa
from expert_ffn_amd import _abi
from oracle import treesel
from synth import routing


def _random_pool(rng, V, L, N, m):
    parent = [-1] + [int(rng.integers(0, v)) for v in range(1, V + 1)]
    level = [0] * (V + 1)
    for v in range(1, V + 1):
        level[v] = level[parent[v]] + 1
    ids = np.array([[rng.choice(N, size=m, replace=False) for _ in range(L)] for _ in range(V + 1)])
    p = [0.0] + [int(rng.integers(0, 9)) / 8 for _ in range(V)]
    return parent, level, ids, p


@pytest.mark.parametrize("seed", range(12))
def test_tree_select_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    V, L, N, m = int(rng.integers(1, 12)), int(rng.integers(1, 4)), int(rng.integers(4, 130)), 0
    m = int(rng.integers(1, min(N, 6) + 1))
    K = int(rng.integers(0, 6))
    parent, level, ids, p = _random_pool(rng, V, L, N, m)
    b = [int(rng.integers(8, 200)) / 8 for _ in range(K + 1)]
    beta = int(rng.integers(1, 16)) / 8
    experts = [[set(ids[v, l].tolist()) for l in range(L)] for v in range(V + 1)]
    for ml in (0, 1, 2):
        lv = None if ml == 0 else level
        S, R, F, T = treesel.select(parent, [Fr(x) for x in p], experts, K, [Fr(x) for x in b], Fr(beta),
                                    None if ml == 0 else ml, lv)
        got = efa.tree_select(parent, p, efa.expert_bitmaps(ids, N), K, b, beta, max_level=ml, level=lv)
        assert got["ids"] == S and got["F"] == F and got["R"] == float(R) and got["T"] == float(T), (ml, got, S)


def _count_legal(parent, K):
    """Ancestor-closed subsets of size <= K, by a tree knapsack (independent of the search)."""
    V = len(parent) - 1
    children = {v: [w for w in range(1, V + 1) if parent[w] == v] for v in range(V + 1)}

    @lru_cache(maxsize=None)
    def closed(v):  # subtrees rooted at v that contain v, by size
        poly = [0, 1]
        for c in children[v]:
            cp = [1] + list(closed(c))[1:]  # c absent, or a subtree rooted at c
            new = [0] * (len(poly) + len(cp) - 1)
            for i, a in enumerate(poly):
                for j, bb in enumerate(cp):
                    if i + j <= K + 1:
                        new[i + j] += a * bb
            poly = new
        return tuple(poly[:K + 2])
    root = closed(0)  # the root counts as one node
    return sum(root[1:K + 2])


def test_tree_workload_enumerates_each_legal_subtree_once():
    parent, tr = routing.tree_routing(128, 8, 0.5, routing.rng_for(5, 0, "tree"))
    ids = tr.ids[:, None, :]  # one layer
    p = [0.0] + [0.5] * 31
    for K in (0, 1, 3, 7):
        got = efa.tree_select(parent, p, efa.expert_bitmaps(ids, 128), K, [1.0] * (K + 1), 0.125)
        assert got["visited"] == _count_legal(list(parent), K)


def test_tree_select_rejects_bad_input():
    bm = np.zeros((3, 1, 1), np.uint64)
    with pytest.raises(_abi.MoeError):  # a parent after its child
        efa.tree_select([-1, 2, 0], [0, 0.5, 0.5], bm, 2, [1, 1, 1], 1)
    with pytest.raises(_abi.MoeError):  # non-positive beta
        efa.tree_select([-1, 0, 1], [0, 0.5, 0.5], bm, 2, [1, 1, 1], 0)
