"""Helpers of the GPU parity tests: build device layers from the seeded inputs,
run both kernels through the C ABI, and compare with the oracle."""
import sys

import numpy as np
import torch

import expert_ffn_amd as efa
import oracle
import synth
from synth.device import to_torch

REL_L2_TOL = 5e-3   # relative L2 error bound on y (bf16 weights, fp32 accumulate)
MAX_ABS_TOL = 3e-2  # max abs error bound on y
SYNC_BYTES = 4 * 32 * (256 + 1024 + 512)  # counter area at the start of a workspace
SUMMATION_TOL = 1e-4  # rel-L2 between per-slot and dedup results (fp32 summation order)


# weight layouts: as given, W_down packed, all three tiled
LAYOUTS = ("plain", "packed", "tiled")


def step_multiple(v, dtype):
    """v rounded up to a whole 64-byte step of the dtype (the tiled layout's unit)."""
    step = 32 if dtype == "bf16" else 16
    return -(-v // step) * step


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


class DeviceLayer:
    """Host weights (for the oracle) and their device copy (for the kernels).  With
    shared experts: ``shared_dev`` holds them as a layer of their own (m = N =
    n_shared, run as a second call) and ``fused`` the routed and shared experts as
    one layer (one call)."""

    def __init__(self, spec, seed, layer=0, with_shared=False, host=None, packed=False, layout=None):
        layout = layout or ("packed" if packed else "plain")
        assert layout in LAYOUTS, layout
        self.layout = layout
        self.spec = spec
        self.host = host if host is not None else synth.layer_weights(spec, seed, layer)
        self.dev = efa.Layer(*(to_torch(a) for a in self.host), m=spec.m)
        self.shared_host = None
        self.shared_dev = None
        self.fused = None
        if with_shared and spec.n_shared:
            self.shared_host = synth.layer_weights(spec, seed, layer, shared=True)
            self.shared_dev = efa.Layer(*(to_torch(a) for a in self.shared_host), m=spec.n_shared)
            sd = self.shared_dev
            self.fused = efa.Layer(self.dev.w_gate, self.dev.w_up, self.dev.w_down, m=spec.m,
                                   shared=(sd.w_gate, sd.w_up, sd.w_down))
        if layout != "plain":  # W_down packed (moe_pack_w_down) or all three tiled (moe_pack_tiled)
            cp = (lambda L: L.packed_copy()) if layout == "packed" else (lambda L: L.tiled_copy())
            self.dev = cp(self.dev)
            if self.fused is not None:
                self.fused = cp(self.fused)
                self.shared_dev = cp(self.shared_dev)
            torch.cuda.synchronize()

    def run(self, x_host, ids_host, w_host, shared=False, stream=None):
        """Returns (y_perslot, y_dedup, info_dedup) on the host; info = (U, ids status, sync status).
        shared: False (routed experts only), "separate" (a second, accumulating call on
        the shared experts' own layer) or "fused" (one call with the shared experts)."""
        x = to_torch(x_host)
        ids = torch.from_numpy(np.ascontiguousarray(ids_host, np.int32)).cuda()
        w = torch.from_numpy(np.ascontiguousarray(w_host, np.float32)).cuda()
        n = x.shape[0]
        layer = self.fused if shared == "fused" else self.dev
        ws = layer.workspace(n)
        info_s = torch.full((3,), 99, dtype=torch.int32, device="cuda")
        info_d = torch.full((3,), 99, dtype=torch.int32, device="cuda")
        ys = efa.expert_perslot(layer, x, ids, w, ws=ws, info=info_s, stream=stream)
        yd = efa.expert_dedup(layer, x, ids, w, ws=ws, info=info_d, stream=stream)
        if shared == "separate":
            E = self.spec.n_shared
            sids = torch.arange(E, dtype=torch.int32, device="cuda").repeat(n, 1).contiguous()
            sw = torch.ones(n, E, dtype=torch.float32, device="cuda")
            sws = self.shared_dev.workspace(n)
            efa.expert_dedup(self.shared_dev, x, sids, sw, y=ys, ws=sws, accumulate=True, stream=stream)
            efa.expert_dedup(self.shared_dev, x, sids, sw, y=yd, ws=sws, accumulate=True, stream=stream)
        torch.cuda.synchronize()
        info_s, info_d = info_s.cpu().numpy(), info_d.cpu().numpy()
        assert np.array_equal(info_s, info_d), (info_s, info_d)
        assert info_d[2] == 0, "internal wait expired"
        assert np.all(ws[:SYNC_BYTES].cpu().numpy() == 0), "sync words not reset"
        return ys.cpu().numpy(), yd.cpu().numpy(), info_d

    def oracle_y(self, x_host, ids_host, w_host, shared=False, tokens=None):
        """fp32 oracle output, for all tokens or the listed ones."""
        if tokens is not None:
            x_host, ids_host, w_host = x_host[tokens], ids_host[tokens], w_host[tokens]
        sh = self.shared_host if shared else None
        return oracle.moe_ffn(*self.host, x_host, ids_host, w_host, self.spec.dtype, shared=sh)


def errors(y, ref):
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    rel = np.linalg.norm(y - ref) / max(np.linalg.norm(ref), 1e-30)
    mx = float(np.max(np.abs(y - ref))) if y.size else 0.0
    return rel, mx


def assert_close(y, ref, what=""):
    rel, mx = errors(y, ref)
    assert np.all(np.isfinite(y)), what
    assert rel <= REL_L2_TOL and mx <= MAX_ABS_TOL, "%s rel_l2=%.3e max_abs=%.3e" % (what, rel, mx)
    return rel, mx


class TorchGenLayer:
    """A full-size layer whose plain weights are drawn on the device by the seeded
    device generator (``synth.device.device_layer_weights``); the kernels run on the
    copies the library's packing kernels make (``layouts``), the oracle on the plain
    weights of the experts a pass touches, copied to the host."""

    def __init__(self, spec, seed, layer=0, layouts=("tiled",), keep_plain=True):
        from synth.device import device_layer_weights
        self.spec = spec
        w = device_layer_weights(spec, seed, layer)
        plain = efa.Layer(*w, m=spec.m)
        self.devs = {}
        for lay in layouts:
            self.devs[lay] = plain if lay == "plain" else (plain.tiled_copy() if lay == "tiled" else plain.packed_copy())
        self.plain = w if keep_plain else None
        self._host = {}
        torch.cuda.synchronize()

    def host_experts(self, experts):
        """(W_gate, W_up, W_down) bf16 bit patterns of the listed experts, [E'][...]."""
        from synth.device import from_torch_bf16
        idx = torch.as_tensor(np.asarray(experts, np.int64), device="cuda")
        return tuple(from_torch_bf16(t.index_select(0, idx)) for t in self.plain)

    def oracle_tasks(self, passes):
        """Arguments of one oracle call per pass (x_host, ids, w), on the experts the
        passes touch only (copied once; each pass's ids renumbered into them)."""
        ex = np.unique(np.concatenate([np.asarray(ids, np.int32).reshape(-1) for _, ids, _ in passes]))
        W = self.host_experts(ex)
        return [(W, np.ascontiguousarray(x), np.searchsorted(ex, np.asarray(ids, np.int32)).astype(np.int32),
                 np.ascontiguousarray(w, np.float32)) for x, ids, w in passes]


def oracle_many(tasks, threads=16):
    """oracle.moe_ffn over many (weights, x, ids, w) tasks on a thread pool (the C call
    releases the GIL); results in task order."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(threads) as pool:
        return list(pool.map(lambda t: oracle.moe_ffn(*t[0], t[1], t[2], t[3], "bf16"), tasks))


def run_pair(layer, x, ids, w, ws, y_slot=None, y_dedup=None):
    """Both kernels on one pass (device tensors) through the C ABI; returns their
    outputs and info words (U, ids status, sync status)."""
    info_s = torch.full((3,), 99, dtype=torch.int32, device="cuda")
    info_d = torch.full((3,), 99, dtype=torch.int32, device="cuda")
    ys = efa.expert_perslot(layer, x, ids, w, y=y_slot, ws=ws, info=info_s)
    yd = efa.expert_dedup(layer, x, ids, w, y=y_dedup, ws=ws, info=info_d)
    return ys, yd, info_s, info_d
