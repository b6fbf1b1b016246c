"""Router of an MoE layer (test infrastructure only).

Lan, arXiv:2610.34440, Section 1: a router sends each token to m of the N experts.
Reading of its steps (the routing weights of the traces, and the plain reading of a
softmax router with top-m): logits l_te = W_r[e] . x_t; the m largest logits of
the token in descending order, equal logits to the lower id; weights = softmax of
the m selected logits (equal to a softmax over all N renormalised to the m).
Everything in float64 from the bf16 (or fp32) values of W_r and x.
"""
import numpy as np


def _f64(a, dtype):
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def logits(w_router, x, dtype):
    """[n][N] float64: l_te = sum_i W_r[e][i] x_t[i] (matmul as the library primitive)."""
    return _f64(x, dtype) @ _f64(w_router, dtype).T


def select(lg, m):
    """ids [n][m]: per row the m largest values, descending, ties to the lower id."""
    lg = np.asarray(lg)
    n, N = lg.shape
    ids = np.empty((n, m), np.int32)
    for t in range(n):
        order = sorted(range(N), key=lambda e: (-lg[t, e], e))
        ids[t] = order[:m]
    return ids


def weights(lg, ids):
    """Softmax of the selected logits, float64 [n][m]."""
    sel = np.take_along_axis(np.asarray(lg, np.float64), np.asarray(ids, np.int64), axis=1)
    ex = np.exp(sel - sel.max(axis=1, keepdims=True))
    return ex / ex.sum(axis=1, keepdims=True)


def route(w_router, x, m, dtype):
    """(ids, w, logits) of a pass."""
    lg = logits(w_router, x, dtype)
    ids = select(lg, m)
    return ids, weights(lg, ids), lg
