"""GPU parity at full size, every output compared with the oracle.

* The Mixtral-shaped layer (N = 8, top-2, d = 4096, d_ff = 14336) under uniform and
  repeat-0.6 routing, n = 1..8, every token, in all three weight layouts.  At n <= 2
  its streaming down items cut the d_ff contraction into parts; that path is here.
* The Qwen3-shaped layer x48 pass in the launch configuration the bench times: 48
  layers, each with its own weights, Zipf routing and activations, tiled weights,
  one workspace, the 48 launches of each kernel back to back on one stream; at
  n = 1, 3 and 8, every layer's output compared.

Weights come from the seeded device generator; the oracle runs on the plain weights
of the experts a pass touches, copied to the host, and the kernels on the copies the
library's packing kernels make.  Bar as in test_gpu_parity.
"""
import numpy as np
import pytest
import torch

import expert_ffn_amd as efa
import oracle
import synth
from synth import routing
from synth.device import to_torch

from .gpu_cases import (SUMMATION_TOL, SYNC_BYTES, TorchGenLayer, assert_close, errors, oracle_many, run_pair,
                        say)

pytestmark = pytest.mark.gpu


def _dev(x, ids, w):
    return (to_torch(x), torch.from_numpy(np.ascontiguousarray(ids, np.int32)).cuda(),
            torch.from_numpy(np.ascontiguousarray(w, np.float32)).cuda())


@pytest.fixture(scope="module")
def mixtral():
    say("mixtral layer from the device generator: plain, packed, tiled")
    return TorchGenLayer(synth.CONFIGS["mixtral"], 9, layouts=("plain", "packed", "tiled"))


@pytest.mark.parametrize("kind", ["uniform", "correlated"])
def test_mixtral_every_token(mixtral, kind):
    spec = mixtral.spec
    tr = routing.make_trace(spec, kind, 256, seed=9, p=0.6)
    starts = routing.window_starts(256, 8, 8, seed=19)
    passes = []
    for n in range(1, 9):
        ids, w = routing.window(tr, int(starts[n - 1]), n)
        passes.append((synth.pass_x(spec, 9, 0, 50 + n, n), ids, w))
    say("mixtral", kind, "oracle of n = 1..8")
    refs = oracle_many(mixtral.oracle_tasks(passes))
    for layout, layer in mixtral.devs.items():
        ws = layer.workspace(8)
        for (x, ids, w), ref in zip(passes, refs):
            n = x.shape[0]
            say("mixtral", kind, layout, "n", n)
            ys, yd, i_s, i_d = run_pair(layer, *_dev(x, ids, w), ws)
            torch.cuda.synchronize()
            assert int(i_d[0]) == oracle.union_count(ids, spec.N) and int(i_d[1]) == 0 and int(i_d[2]) == 0
            assert int(i_s[2]) == 0
            assert_close(ys.cpu().numpy(), ref, "mixtral %s %s n=%d perslot" % (kind, layout, n))
            assert_close(yd.cpu().numpy(), ref, "mixtral %s %s n=%d dedup" % (kind, layout, n))
            assert errors(ys.cpu().numpy(), yd.cpu().numpy())[0] <= SUMMATION_TOL
        assert np.all(ws[:SYNC_BYTES].cpu().numpy() == 0)


def test_qwen3x48_full_pass_every_layer():
    spec = synth.CONFIGS["qwen3"]
    L, T, seed = spec.layers, 512, 51
    ns = (1, 3, 8)
    traces = [routing.make_trace(spec, "zipf", T, seed=seed, layer=l, s=1.1) for l in range(L)]
    starts = {n: int(routing.window_starts(T, n, 1, seed=seed)[0]) for n in ns}
    layers, tasks = [], []
    from concurrent.futures import ThreadPoolExecutor
    pool = ThreadPoolExecutor(16)
    for l in range(L):
        if l % 8 == 0:
            say("qwen3 x48: layer", l, "from the device generator, tiled; oracle tasks queued")
        g = TorchGenLayer(spec, seed, layer=l, layouts=("tiled",))
        passes = []
        for n in ns:
            ids, w = routing.window(traces[l], starts[n], n)
            passes.append((synth.pass_x(spec, seed, l, n, n), ids, w))
        tasks.append(pool.submit(oracle_many, g.oracle_tasks(passes), 1))
        g.plain = None
        layers.append((g.devs["tiled"], passes))
    ws = layers[0][0].workspace(8)
    for ni, n in enumerate(ns):
        say("qwen3 x48: n", n, "48 launches per kernel back to back")
        dev = [_dev(*layers[l][1][ni]) for l in range(L)]
        ys = torch.empty(L, n, spec.d, dtype=torch.float32, device="cuda")
        yd = torch.empty_like(ys)
        info = torch.full((L, 2, 3), 99, dtype=torch.int32, device="cuda")
        for l in range(L):
            efa.expert_perslot(layers[l][0], *dev[l], y=ys[l], ws=ws, info=info[l, 0])
        for l in range(L):
            efa.expert_dedup(layers[l][0], *dev[l], y=yd[l], ws=ws, info=info[l, 1])
        torch.cuda.synchronize()
        inf = info.cpu().numpy()
        ys_h, yd_h = ys.cpu().numpy(), yd.cpu().numpy()
        for l in range(L):
            ref = tasks[l].result()[ni]
            x, ids, w = layers[l][1][ni]
            assert inf[l, 1, 0] == oracle.union_count(ids, spec.N) and inf[l, 1, 1] == 0
            assert inf[l, 0, 2] == 0 and inf[l, 1, 2] == 0
            assert_close(ys_h[l], ref, "qwen3x48 n=%d layer %d perslot" % (n, l))
            assert_close(yd_h[l], ref, "qwen3x48 n=%d layer %d dedup" % (n, l))
            assert errors(ys_h[l], yd_h[l])[0] <= SUMMATION_TOL
    assert np.all(ws[:SYNC_BYTES].cpu().numpy() == 0)
    pool.shutdown()
