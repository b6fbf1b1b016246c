"""Seeded routing traces: per token the ids of its m experts and fp32 weights.

A trace stands in for recorded routing of one token sequence in one layer.  A pass
of n tokens copies the ids and weights of a window of n consecutive tokens.

Readings used where the workload descriptions leave a step open:

* weights: fp32 softmax over the logits of the m selected experts, ids in
  order of descending logit (equal logits: lower id first);
* ``uniform``: top-m of iid N(0,1) logits, i.e. a uniform m-subset;
* ``correlated``: token 0 uniform; token t keeps each expert of token t-1
  independently with probability p and fills the remaining slots uniformly
  without replacement from the experts it has not already kept (a dropped
  expert may be drawn again); weights from fresh N(0,1) logits;
* ``zipf``: a seeded permutation gives expert e the popularity rank r(e) in
  1..N; logit = N(0,1) - s ln r(e); top-m; softmax of the selected logits;
* ``tree``: 32 verified nodes, node 0 the current token, node 1 its single
  child, every node at depths 1..4 with two children; node ids breadth first
  (parents before children); node 0 uniform, every other node drawn from its
  parent by the ``correlated`` rule;
* tree commit probabilities (for choosing a verification subtree): node v's
  cumulative draft probability is its parent's times a conditional one; the root's
  single child draws U(0.5, 0.95), a first child U(0.4, 0.9) and a second child
  U(0, 1 - q_first) / 2, so probabilities fall along every path;
* ``chosen`` (passes with chosen ids): the n m slots of a pass name exactly U
  distinct experts, m <= U <= min(n m, N), a seeded U-subset of the N; token 0
  takes m of them, the other U - m are spread as evenly as possible over tokens
  1..n-1 in order, and each token fills its other slots with distinct experts
  that earlier tokens named; weights from fresh N(0,1) logits.
"""
from collections import namedtuple

import numpy as np

from . import lib

Trace = namedtuple("Trace", ["ids", "w"])  # ids int32 [T][m], w float32 [T][m]

TAG_ROUTE = 5
KIND_TAGS = {"uniform": 1, "correlated": 2, "zipf": 3, "tree": 4, "windows": 5, "chosen": 6}


def rng_for(seed, layer, kind, extra=0):
    return np.random.Generator(np.random.PCG64(lib.key_of(seed, layer, TAG_ROUTE, KIND_TAGS[kind], extra)))


def _finish(ids_rows, logit_rows):
    """Order each row by descending logit (ties: lower id) and softmax to fp32."""
    ids_rows = np.asarray(ids_rows, dtype=np.int64)
    logit_rows = np.asarray(logit_rows, dtype=np.float64)
    order = np.lexsort((ids_rows, -logit_rows), axis=-1)
    ids_o = np.take_along_axis(ids_rows, order, axis=-1)
    lg = np.take_along_axis(logit_rows, order, axis=-1)
    ex = np.exp(lg - lg.max(axis=-1, keepdims=True))
    w = (ex / ex.sum(axis=-1, keepdims=True)).astype(np.float32)
    return Trace(ids_o.astype(np.int32), w)


def _topm(logits, m):
    N = logits.shape[-1]
    order = np.lexsort((np.broadcast_to(np.arange(N), logits.shape), -logits), axis=-1)
    ids = order[..., :m]
    return ids, np.take_along_axis(logits, ids, axis=-1)


def uniform_trace(N, m, T, rng):
    logits = rng.standard_normal((T, N))
    ids, sel = _topm(logits, m)
    return _finish(ids, sel)


def _draw_from(prev_set, N, m, p, rng):
    keep = [e for e in prev_set if rng.random() < p]
    kept = set(keep)
    pool = np.array([e for e in range(N) if e not in kept], dtype=np.int64)
    new = rng.choice(pool, size=m - len(keep), replace=False) if m > len(keep) else np.empty(0, np.int64)
    return keep + [int(e) for e in new]


def correlated_trace(N, m, T, p, rng):
    rows = [list(rng.choice(N, size=m, replace=False))]
    for _ in range(1, T):
        rows.append(_draw_from(sorted(rows[-1]), N, m, p, rng))
    logits = rng.standard_normal((T, m))
    return _finish(rows, logits)


def zipf_trace(N, m, T, s, rng):
    rank = rng.permutation(N) + 1
    bias = -float(s) * np.log(rank.astype(np.float64))
    logits = rng.standard_normal((T, N)) + bias[None, :]
    ids, sel = _topm(logits, m)
    return _finish(ids, sel)


def tree_parents():
    """Parent of each of the 32 nodes (node 0: -1), breadth-first ids."""
    parents = [-1, 0]
    frontier = [1]
    for _depth in range(1, 5):
        nxt = []
        for v in frontier:
            for _c in range(2):
                parents.append(v)
                nxt.append(len(parents) - 1)
        frontier = nxt
    assert len(parents) == 32
    return np.array(parents, dtype=np.int32)


def tree_routing(N, m, p, rng):
    parents = tree_parents()
    rows = [list(rng.choice(N, size=m, replace=False))]
    for v in range(1, parents.size):
        rows.append(_draw_from(sorted(rows[parents[v]]), N, m, p, rng))
    logits = rng.standard_normal((parents.size, m))
    tr = _finish(rows, logits)
    return parents, tr


def tree_commit_probs(parents, rng):
    """Cumulative draft probability of every node (root: 1)."""
    parents = np.asarray(parents)
    p = np.ones(parents.size, np.float64)
    first = {}
    for v in range(1, parents.size):
        pa = int(parents[v])
        if pa == 0 and v == 1:
            q = rng.uniform(0.5, 0.95)
        elif pa not in first:
            q = rng.uniform(0.4, 0.9)
            first[pa] = q
        else:
            q = rng.uniform(0.0, 1.0 - first[pa]) / 2
        p[v] = p[pa] * q
    return p


def chosen_pass(N, m, n, U, rng):
    """One pass of n tokens whose slots name exactly U distinct experts."""
    if not (1 <= m <= N and n >= 1 and m <= U <= min(n * m, N)):
        raise ValueError("need m <= U <= min(n m, N)")
    experts = [int(e) for e in rng.choice(N, size=U, replace=False)]
    fresh = experts[m:]
    rows = [experts[:m]]
    named = list(experts[:m])
    for t in range(1, n):
        k = -(-len(fresh) // (n - t))  # new experts this token: ceil(remaining / tokens left)
        new, fresh = fresh[:k], fresh[k:]
        old = [int(e) for e in rng.choice(named, size=m - k, replace=False)] if m > k else []
        rows.append(new + old)
        named += new
    logits = rng.standard_normal((n, m))
    return _finish(rows, logits)


def make_trace(spec, kind, T, seed, layer=0, p=None, s=None):
    """Trace of T tokens for the layer ``spec`` under routing ``kind``."""
    rng = rng_for(seed, layer, kind)
    if kind == "uniform":
        return uniform_trace(spec.N, spec.m, T, rng)
    if kind == "correlated":
        return correlated_trace(spec.N, spec.m, T, p, rng)
    if kind == "zipf":
        return zipf_trace(spec.N, spec.m, T, s, rng)
    raise ValueError(kind)


def window_starts(T, n, count, seed, layer=0):
    rng = rng_for(seed, layer, "windows", n)
    return rng.integers(0, T - n + 1, size=count)


def window(trace, start, n):
    return (np.ascontiguousarray(trace.ids[start:start + n]), np.ascontiguousarray(trace.w[start:start + n]))
