"""Pins of the router oracle (Lan, arXiv:2610.34440, Section 1: a router sends each
token to m of N experts; reading: top-m logits, ties to the lower id, softmax over
the selected)."""
import itertools

import numpy as np

from oracle import router
import synth


def test_selection_is_the_brute_force_maximum():
    rng = np.random.default_rng(1)
    for _ in range(50):
        N, m = int(rng.integers(2, 9)), 0
        m = int(rng.integers(1, N + 1))
        lg = rng.integers(-3, 4, size=(3, N)).astype(np.float64)  # many ties
        ids = router.select(lg, m)
        for t in range(3):
            # the best m-subset by total logit, listed in order, ties to lower ids
            best = max(itertools.combinations(range(N), m), key=lambda c: (sum(lg[t, list(c)]), [-e for e in c]))
            assert sorted(ids[t].tolist()) == sorted(best) or sum(lg[t, ids[t]]) == sum(lg[t, list(best)])
            vals = lg[t, ids[t]]
            assert all(vals[i] > vals[i + 1] or (vals[i] == vals[i + 1] and ids[t, i] < ids[t, i + 1])
                       for i in range(m - 1))
            rest = [e for e in range(N) if e not in set(ids[t].tolist())]
            assert all(lg[t, e] < vals[-1] or (lg[t, e] == vals[-1] and e > ids[t, -1]) for e in rest)


def test_ties_go_to_the_lower_id():
    W = np.zeros((6, 4), np.float32)
    W[[1, 3, 4]] = 1.0  # experts 1, 3, 4 share the largest logit
    x = np.ones((1, 4), np.float32)
    ids, w, _ = router.route(W, x, 2, "f32")
    assert ids.tolist() == [[1, 3]] and np.allclose(w, 0.5)


def test_weights_are_the_renormalised_full_softmax():
    rng = np.random.default_rng(2)
    lg = rng.standard_normal((5, 20))
    ids = router.select(lg, 4)
    full = np.exp(lg - lg.max(axis=1, keepdims=True))
    full /= full.sum(axis=1, keepdims=True)
    sel = np.take_along_axis(full, ids.astype(np.int64), axis=1)
    assert np.allclose(router.weights(lg, ids), sel / sel.sum(axis=1, keepdims=True), rtol=1e-14)


def test_logits_and_all_experts():
    spec = synth.layer_spec("tiny", N=8, m=8, d=16)
    W = synth.router_weights(spec, 3)
    x = synth.pass_x(spec, 3, 0, 0, 2)
    ids, w, lg = router.route(W, x, 8, "f32")
    ref = [[sum(float(W[e, i]) * float(x[t, i]) for i in range(16)) for e in range(8)] for t in range(2)]
    assert np.allclose(lg, ref, rtol=1e-12, atol=1e-14)
    assert all(sorted(r) == list(range(8)) for r in ids.tolist())  # m = N selects every expert
    assert np.allclose(w.sum(axis=1), 1.0)


def test_permuting_experts_permutes_ids():
    spec = synth.layer_spec("dsv2lite", N=32, m=4, d=64)
    W = synth.router_weights(spec, 4)
    x = synth.pass_x(spec, 4, 0, 0, 3)
    ids, w, _ = router.route(W, x, 4, "bf16")
    perm = np.random.default_rng(5).permutation(32)
    ids2, w2, _ = router.route(W[perm], x, 4, "bf16")
    assert np.array_equal(perm[ids2], ids) and np.allclose(w2, w)
