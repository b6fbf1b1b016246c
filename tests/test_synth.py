"""Checks of the seeded input generators (they feed both the GPU path and the oracle)."""
import math
from math import comb

import numpy as np
import pytest
import torch

import synth
from oracle import reuse
from synth import lib, routing


def test_counter_based_stream_matches_definition():
    key = lib.key_of(1, 2, 3)
    got = lib.normal_f64(key, 6, start=3)
    for j in range(6):
        i = 3 + j
        p = i // 2
        x0 = lib.mix64(key + (2 * p + 1) * lib.GOLDEN)
        x1 = lib.mix64(key + (2 * p + 2) * lib.GOLDEN)
        u1 = ((x0 >> 11) + 1) * 2.0 ** -53
        u2 = (x1 >> 11) * 2.0 ** -53
        r = math.sqrt(-2 * math.log(u1))
        z = r * (math.sin(2 * math.pi * u2) if i % 2 else math.cos(2 * math.pi * u2))
        assert abs(got[j] - z) < 1e-12


def test_normal_moments_and_bf16_rounding():
    v = lib.normal_f32(lib.key_of(9), 2_000_000, 0.02)
    assert abs(v.mean()) < 1e-4 and abs(v.std() - 0.02) < 1e-4
    b = lib.normal_bf16(lib.key_of(9), 2_000_000, 0.02)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b, ref)  # round-to-nearest-even, as torch does
    assert np.array_equal(lib.f32_to_bf16(v), ref)


def test_expert_weights_regenerate_alone():
    spec = synth.layer_spec("dsv2lite", N=4, d=64, d_ff=48)
    Wg, Wu, Wd = synth.layer_weights(spec, 5)
    g, u, d = synth.expert_weights(spec, 5, 0, 2)
    assert np.array_equal(Wg[2], g) and np.array_equal(Wu[2], u) and np.array_equal(Wd[2], d)
    assert not np.array_equal(Wg[1], Wg[2])


def test_uniform_trace_is_uniform_subsets():
    tr = routing.uniform_trace(8, 2, 20000, routing.rng_for(1, 0, "uniform"))
    assert tr.ids.dtype == np.int32 and tr.w.dtype == np.float32
    for row in tr.ids[:100]:
        assert len(set(row.tolist())) == 2
    cnt = np.bincount(tr.ids.reshape(-1), minlength=8) / (2 * 20000)
    assert np.all(np.abs(cnt - 1 / 8) < 0.01)
    np.testing.assert_allclose(tr.w.sum(axis=1), 1, rtol=1e-6)
    assert np.all(np.diff(tr.w, axis=1) <= 0)  # descending logit order


def _rho2_exact(N, m, p):
    """(1/m) E[K + (m-K)^2/(N-K)], K ~ Bin(m, p): next-token reuse of the correlated rule."""
    s = 0.0
    for K in range(m + 1):
        pk = comb(m, K) * p ** K * (1 - p) ** (m - K)
        s += pk * (K + (m - K) ** 2 / (N - K))
    return s / m


def test_correlated_trace_next_token_reuse():
    for N, m, p, want in [(64, 6, 0.5, 0.5283), (8, 2, 0.6, 0.6743)]:
        tr = routing.correlated_trace(N, m, 30000, p, routing.rng_for(2, 0, "correlated"))
        exact = _rho2_exact(N, m, p)
        assert abs(exact - want) < 1e-4
        assert abs(reuse.rho_hat(tr.ids, 2, m) - exact) < 0.01
        for row in tr.ids[:200]:
            assert len(set(row.tolist())) == m


def test_zipf_trace_skews_popularity():
    tr = routing.zipf_trace(128, 8, 4096, 1.1, routing.rng_for(3, 0, "zipf"))
    cnt = np.sort(np.bincount(tr.ids.reshape(-1), minlength=128))[::-1]
    assert cnt[0] > 5 * cnt[64]


def test_tree_shape():
    par = routing.tree_parents()
    assert par.size == 32 and par[0] == -1 and par[1] == 0
    depth = [0] * 32
    for v in range(1, 32):
        assert par[v] < v
        depth[v] = depth[par[v]] + 1
    assert [depth.count(k) for k in range(6)] == [1, 1, 2, 4, 8, 16]
    _, tr = routing.tree_routing(128, 8, 0.5, routing.rng_for(4, 0, "tree"))
    assert tr.ids.shape == (32, 8)


def test_chosen_passes_name_exactly_U_experts():
    from synth import routing
    rng = routing.rng_for(3, 0, "chosen")
    for N, m, n in ((64, 6, 1), (64, 6, 2), (64, 6, 9), (8, 2, 4), (128, 8, 8), (10, 3, 5)):
        for U in range(m, min(n * m, N) + 1):
            tr = routing.chosen_pass(N, m, n, U, rng)
            assert tr.ids.shape == (n, m) and tr.w.shape == (n, m)
            assert len(set(tr.ids.reshape(-1).tolist())) == U
            assert all(len(set(r)) == m for r in tr.ids.tolist())
            assert tr.ids.min() >= 0 and tr.ids.max() < N
            assert np.allclose(tr.w.sum(axis=1), 1.0, atol=1e-6)
    with pytest.raises(ValueError):
        routing.chosen_pass(64, 6, 2, 5, rng)
    with pytest.raises(ValueError):
        routing.chosen_pass(8, 2, 8, 9, rng)
