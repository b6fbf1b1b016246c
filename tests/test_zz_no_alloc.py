"""moe_expert_auto_noalloc, the entry point that allocates nothing (its workspace is
the library's per-GPU scratch array), against moe_expert_auto with a caller
workspace: the same kernel runs and gives the same bits, on two calls in a row, the
second with a smaller pass; both within the oracle bar.  On the CPU: a pass larger
than the array and a negative crossover are refused before anything is launched."""
import ctypes

import numpy as np
import pytest
import torch

import expert_ffn_amd as efa
import synth
from expert_ffn_amd import _abi
from synth import routing
from synth.device import to_torch

from .gpu_cases import SYNC_BYTES, DeviceLayer, TorchGenLayer, assert_close, oracle_many, say


def _dev(x, ids, w):
    return (to_torch(x), torch.from_numpy(np.ascontiguousarray(ids, np.int32)).cuda(),
            torch.from_numpy(np.ascontiguousarray(w, np.float32)).cuda())


def _two_calls(layer, ws, passes, crossover, refs):
    for (x_h, ids_h, w_h), ref in zip(passes, refs):
        n = x_h.shape[0]
        x, ids, w = _dev(x_h, ids_h, w_h)
        say("noalloc crossover", crossover, "n", n)
        y_ref, k_ref = efa.expert_auto(layer, x, ids, w, crossover, ws=ws)
        y = torch.full((n, layer.d), float("nan"), dtype=torch.float32, device="cuda")
        info = torch.full((3,), 99, dtype=torch.int32, device="cuda")
        y2, k = efa.expert_auto_noalloc(layer, x, ids, w, crossover, y=y, info=info)
        torch.cuda.synchronize()
        assert y2.data_ptr() == y.data_ptr()
        assert k == k_ref == (efa.MOE_KIND_DEDUP if (crossover > 0 and n >= crossover) else efa.MOE_KIND_SLOT)
        assert torch.equal(y, y_ref), "noalloc differs from the workspace call (n=%d)" % n
        inf = info.cpu().numpy()
        assert inf[0] == len(set(np.asarray(ids_h).reshape(-1).tolist())) and inf[1] == 0 and inf[2] == 0
        assert_close(y.cpu().numpy(), ref, "noalloc n=%d crossover %d" % (n, crossover))


@pytest.mark.gpu
@pytest.mark.parametrize("crossover", [0, 1])
def test_noalloc_equals_workspace_call_with_shared_experts(crossover):
    spec = synth.layer_spec("dsv2lite", N=32, m=4, d=512, d_ff=384, n_shared=2)
    dl = DeviceLayer(spec, 61, with_shared=True, layout="tiled")
    tr = routing.make_trace(spec, "correlated", 64, seed=61, p=0.5)
    passes = []
    for n in (8, 3):  # the second call smaller
        ids, w = routing.window(tr, 2 * n, n)
        passes.append((synth.pass_x(spec, 61, 0, n, n), ids, w))
    refs = [dl.oracle_y(x, ids, w, shared=True) for x, ids, w in passes]
    ws = dl.fused.workspace(8)
    _two_calls(dl.fused, ws, passes, crossover, refs)
    assert np.all(ws[:SYNC_BYTES].cpu().numpy() == 0)


@pytest.mark.gpu
@pytest.mark.parametrize("crossover", [0, 2])
def test_noalloc_equals_workspace_call_qwen3_shape(crossover):
    spec = synth.CONFIGS["qwen3"]
    g = TorchGenLayer(spec, 62, layouts=("tiled",))
    layer = g.devs["tiled"]
    tr = routing.make_trace(spec, "zipf", 256, seed=62, s=1.1)
    passes = []
    for n in (8, 2):
        ids, w = routing.window(tr, 5 * n, n)
        passes.append((synth.pass_x(spec, 62, 0, n, n), ids, w))
    refs = oracle_many(g.oracle_tasks(passes))
    _two_calls(layer, layer.workspace(8), passes, crossover, refs)


def test_noalloc_refuses_passes_larger_than_the_array():
    L = _abi.lib()
    # d = d_ff = 16384, n = 64: h and O of 128 slots need more than MOE_SCRATCH_BYTES
    desc = _abi.LayerDesc(8, 2, 16384, 16384, _abi.MOE_BF16, 0, 0)
    assert L.moe_workspace_bytes(ctypes.byref(desc), 64, 0) > _abi.MOE_SCRATCH_BYTES
    wts = _abi.LayerWeights(16, 16, 16, 0, 0, 0)
    kind = ctypes.c_int32(-7)
    for cross in (0, 1):
        st = L.moe_expert_auto_noalloc(ctypes.byref(desc), ctypes.byref(wts), 16, 16, 16, 64, 16, None, cross,
                                       ctypes.byref(kind), None)
        assert st == _abi.MOE_E_WORKSPACE and kind.value == -7
    st = L.moe_expert_auto_noalloc(ctypes.byref(desc), ctypes.byref(wts), 16, 16, 16, 1, 16, None, -1,
                                   ctypes.byref(kind), None)
    assert st == _abi.MOE_E_INVAL and kind.value == -7
