"""The router on the GPU (moe_router_topk) against the oracle (Lan,
arXiv:2610.34440, Section 1: a router sends each token to m of N experts).

Logits within an fp32 summation bound of the float64 oracle; ids bit-exact
against the selection rule applied to the kernel's own fp32 logits, and equal to
the oracle's wherever the oracle's m-th and (m+1)-th logits are further apart
than twice that bound; weights against the float64 softmax of the selected fp32
logits.  A pass routed on the GPU then runs through the expert kernels."""
import numpy as np
import pytest
import torch

import expert_ffn_amd as efa
import synth
from oracle import router as oracle_router
from synth.device import to_torch

from .gpu_cases import DeviceLayer, assert_close, say

pytestmark = pytest.mark.gpu


def _abs_products(W, x, dtype):
    Wf, xf = oracle_router._f64(W, dtype), oracle_router._f64(x, dtype)
    return np.abs(xf) @ np.abs(Wf).T


def _check(spec, W, x, m):
    Wd, xd = to_torch(W), to_torch(x)
    out = efa.router_topk(Wd, xd, m)
    torch.cuda.synchronize()
    lg, ids, w = out.logits.cpu().numpy(), out.ids.cpu().numpy(), out.w.cpu().numpy()
    ref_ids, _, ref_lg = oracle_router.route(W, x, m, spec.dtype)
    bound = 1e-5 * _abs_products(W, x, spec.dtype) + 1e-30
    assert np.all(np.abs(lg - ref_lg) <= bound), float(np.max(np.abs(lg - ref_lg) / bound))
    # the selection rule on the kernel's own fp32 logits
    assert np.array_equal(ids, oracle_router.select(lg.astype(np.float64), m))
    # the oracle's ids where its selection is separated by more than the error
    N = lg.shape[1]
    for t in range(lg.shape[0]):
        srt = np.sort(ref_lg[t])[::-1]
        if m < N and srt[m - 1] - srt[m] > 2 * bound[t].max():
            assert np.array_equal(ids[t], ref_ids[t]), t
    sel = np.take_along_axis(lg.astype(np.float64), ids.astype(np.int64), axis=1)
    ex = np.exp(sel - sel[:, :1])
    assert np.allclose(w, ex / ex.sum(axis=1, keepdims=True), rtol=2e-6, atol=1e-7)
    return out


@pytest.mark.parametrize("base,N,m,d,n", [
    ("dsv2lite", 64, 6, 2048, 1), ("dsv2lite", 64, 6, 2048, 8), ("qwen3", 128, 8, 2048, 17),
    ("qwen3", 128, 8, 2048, 64), ("tiny", 8, 2, 64, 4), ("tiny", 70, 5, 200, 19), ("dsv2lite", 1024, 16, 136, 5),
    ("dsv2lite", 3, 3, 8, 2), ("mixtral", 8, 2, 4096, 8), ("qwen3", 1024, 8, 2048, 64), ("qwen3", 128, 8, 2048, 1)])
def test_router_matches_oracle(base, N, m, d, n):
    spec = synth.layer_spec(base, N=N, m=m, d=d)
    say("router", base, N, m, d, n)
    W = synth.router_weights(spec, 9)
    x = synth.pass_x(spec, 9, 0, 5, n)
    _check(spec, W, x, m)


def test_router_ties_and_repeated_calls():
    spec = synth.layer_spec("dsv2lite", N=40, m=5, d=64)
    W = synth.router_weights(spec, 2)
    W[[3, 17, 30]] = W[11]  # four experts with bit-identical logits
    x = synth.pass_x(spec, 2, 0, 1, 6)
    a = _check(spec, W, x, 5)
    b = _check(spec, W, x, 5)
    assert torch.equal(a.ids, b.ids) and torch.equal(a.w, b.w) and torch.equal(a.logits, b.logits)


@pytest.mark.parametrize("layout,d_ff", [("packed", 176), ("tiled", 192)])
def test_routed_pass_through_the_expert_kernels(layout, d_ff):
    spec = synth.layer_spec("dsv2lite", N=16, m=4, d=256, d_ff=d_ff, n_shared=0)
    dl = DeviceLayer(spec, 12, layout=layout)
    W = synth.router_weights(spec, 12)
    x = synth.pass_x(spec, 12, 0, 3, 7)
    say("routed pass")
    out = efa.router_topk(to_torch(W), to_torch(x), spec.m)
    torch.cuda.synchronize()
    ids, w = out.ids.cpu().numpy(), out.w.cpu().numpy()
    ys, yd, info = dl.run(x, ids, w)
    ref = dl.oracle_y(x, ids, w)
    assert_close(ys, ref, "routed perslot")
    assert_close(yd, ref, "routed dedup")
