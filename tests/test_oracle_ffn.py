"""Pins of the oracle's expert FFN against things other than itself.

The pages print no FFN values, so the oracle's FFN is pinned by
  (i)  a library routine: with N = m = 1 and w = 1 the operation is one SwiGLU MLP,
       compared with PyTorch CPU float64 (F.silu, matmul);
  (ii) a closed form: d_ff = d, W_gate = W_up = alpha I, W_down = I gives
       y = sum_j w_j silu(alpha_j x) alpha_j x elementwise;
  (iii) structure: linearity in the routing weights, token permutation, slot order,
       shared experts as extra weight-1 experts.
Shapes are non-square (d != d_ff) so a transposed operand fails (i).
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

import oracle
import synth
from synth import routing


def _torch_swiglu(wg, wu, wd, x):
    """PyTorch float64 reference: (silu(x Wg^T) * (x Wu^T)) Wd^T."""
    wg, wu, wd, x = (torch.from_numpy(np.asarray(a, np.float64)) for a in (wg, wu, wd, x))
    return (Fn.silu(x @ wg.T) * (x @ wu.T)) @ wd.T


def _dec(a, dtype):
    return synth.bf16_to_f32(a).astype(np.float64) if dtype == "bf16" else np.asarray(a, np.float64)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d,d_ff", [(64, 96), (40, 24)])
def test_single_expert_is_swiglu_mlp(dtype, d, d_ff):
    spec = synth.layer_spec("tiny", N=1, m=1, d=d, d_ff=d_ff, dtype=dtype, sigma=0.2)
    Wg, Wu, Wd = synth.layer_weights(spec, seed=11)
    x = synth.pass_x(spec, 11, 0, 0, 3)
    ids = np.zeros((3, 1), np.int32)
    w = np.ones((3, 1), np.float32)
    got = oracle.moe_ffn_f64(Wg, Wu, Wd, x, ids, w, dtype)
    ref = _torch_swiglu(_dec(Wg[0], dtype), _dec(Wu[0], dtype), _dec(Wd[0], dtype), _dec(x, dtype)).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)


def test_mixture_matches_torch_weighted_sum():
    spec = synth.layer_spec("tiny", N=5, m=3, d=48, d_ff=80, dtype="bf16", sigma=0.1)
    Wg, Wu, Wd = synth.layer_weights(spec, seed=3)
    tr = routing.uniform_trace(5, 3, 4, routing.rng_for(3, 0, "uniform"))
    x = synth.pass_x(spec, 3, 0, 0, 4)
    got = oracle.moe_ffn_f64(Wg, Wu, Wd, x, tr.ids, tr.w, "bf16")
    xd = _dec(x, "bf16")
    ref = np.zeros_like(got)
    for t in range(4):
        for j in range(3):
            e = tr.ids[t, j]
            ref[t] += float(tr.w[t, j]) * _torch_swiglu(_dec(Wg[e], "bf16"), _dec(Wu[e], "bf16"),
                                                        _dec(Wd[e], "bf16"), xd[t:t + 1]).numpy()[0]
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)


def test_identity_weights_closed_form():
    d, n = 16, 3
    alphas = [0.5, -1.25]
    Wg = np.stack([a * np.eye(d, dtype=np.float32) for a in alphas])
    Wd = np.stack([np.eye(d, dtype=np.float32) for _ in alphas])
    x = np.linspace(-3, 3, n * d, dtype=np.float32).reshape(n, d)
    ids = np.tile(np.array([[0, 1]], np.int32), (n, 1))
    w = np.array([[0.75, 0.25], [0.5, 0.5], [1.0, 2.0]], np.float32)
    got = oracle.moe_ffn_f64(Wg, Wg.copy(), Wd, x, ids, w, "f32")
    xd = x.astype(np.float64)
    ref = np.zeros_like(xd)
    for j, a in enumerate(alphas):
        z = a * xd
        ref += w[:, j:j + 1].astype(np.float64) * (z / (1 + np.exp(-z))) * z
    np.testing.assert_allclose(got, ref, rtol=1e-14, atol=1e-15)


def _tiny_case(seed=5, n=4):
    spec = synth.CONFIGS["tiny"]
    W = synth.layer_weights(spec, seed)
    tr = routing.uniform_trace(spec.N, spec.m, n, routing.rng_for(seed, 0, "uniform"))
    x = synth.pass_x(spec, seed, 0, 0, n)
    return spec, W, x, tr.ids, tr.w


def test_linear_in_routing_weights():
    spec, W, x, ids, _ = _tiny_case()
    # dyadic weights so that w + w2 is exact in fp32
    w = (np.arange(ids.size, dtype=np.float32).reshape(ids.shape) + 1) / 8
    w2 = np.flip(w, axis=1).copy() * np.float32(0.5)
    y1 = oracle.moe_ffn_f64(*W, x, ids, w, "f32")
    y2 = oracle.moe_ffn_f64(*W, x, ids, w2, "f32")
    y12 = oracle.moe_ffn_f64(*W, x, ids, (w + w2).astype(np.float32), "f32")
    np.testing.assert_allclose(y12, y1 + y2, rtol=1e-12, atol=1e-15)
    y0 = oracle.moe_ffn_f64(*W, x, ids, np.zeros_like(w), "f32")
    assert np.all(y0 == 0)


def test_token_permutation_and_slot_order():
    spec, W, x, ids, w = _tiny_case(seed=8, n=5)
    y = oracle.moe_ffn_f64(*W, x, ids, w, "f32")
    perm = np.array([3, 0, 4, 1, 2])
    yp = oracle.moe_ffn_f64(*W, x[perm], ids[perm], w[perm], "f32")
    assert np.array_equal(yp, y[perm])
    ys = oracle.moe_ffn_f64(*W, x, ids[:, ::-1].copy(), w[:, ::-1].copy(), "f32")
    np.testing.assert_allclose(ys, y, rtol=1e-13, atol=1e-16)


def test_shared_experts_are_weight_one_experts():
    spec = synth.layer_spec("dsv2lite", N=6, m=2, d=32, d_ff=40, n_shared=2)
    W = synth.layer_weights(spec, 21)
    S = synth.layer_weights(spec, 21, shared=True)
    tr = routing.uniform_trace(6, 2, 3, routing.rng_for(21, 0, "uniform"))
    x = synth.pass_x(spec, 21, 0, 0, 3)
    y = oracle.moe_ffn(*W, x, tr.ids, tr.w, "bf16", shared=S)
    ref = oracle.moe_ffn_f64(*W, x, tr.ids, tr.w, "bf16")
    xd = _dec(x, "bf16")
    for s in range(2):
        ref += _torch_swiglu(_dec(S[0][s], "bf16"), _dec(S[1][s], "bf16"), _dec(S[2][s], "bf16"), xd).numpy()
    np.testing.assert_array_equal(y, ref.astype(np.float32))


def test_invalid_ids_rejected():
    spec, W, x, ids, w = _tiny_case()
    bad = ids.copy()
    bad[1, 0] = spec.N
    with pytest.raises(ValueError):
        oracle.moe_ffn_f64(*W, x, bad, w, "f32")
    dup = ids.copy()
    dup[2, 1] = dup[2, 0]
    with pytest.raises(ValueError):
        oracle.moe_ffn_f64(*W, x, dup, w, "f32")
