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


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


class DeviceLayer:
    """Host weights (for the oracle) and their device copy (for the kernels)."""

    def __init__(self, spec, seed, layer=0, with_shared=False, host=None):
        self.spec = spec
        self.host = host if host is not None else synth.layer_weights(spec, seed, layer)
        self.dev = efa.Layer(*(to_torch(a) for a in self.host), m=spec.m)
        self.shared_host = None
        self.shared_dev = None
        if with_shared and spec.n_shared:
            self.shared_host = synth.layer_weights(spec, seed, layer, shared=True)
            self.shared_dev = efa.Layer(*(to_torch(a) for a in self.shared_host), m=spec.n_shared)

    def run(self, x_host, ids_host, w_host, shared=False, stream=None):
        """Returns (y_perslot, y_dedup, u_and_err) on the host."""
        x = to_torch(x_host)
        ids = torch.from_numpy(np.ascontiguousarray(ids_host, np.int32)).cuda()
        w = torch.from_numpy(np.ascontiguousarray(w_host, np.float32)).cuda()
        ys = efa.expert_perslot(self.dev, x, ids, w, stream=stream)
        grp = efa.route_group(ids, self.spec.N, stream=stream)
        yd = efa.expert_dedup(self.dev, x, ids, w, grp, stream=stream)
        if shared:
            n = x.shape[0]
            E = self.spec.n_shared
            sids = torch.arange(E, dtype=torch.int32, device="cuda").repeat(n, 1).contiguous()
            sw = torch.ones(n, E, dtype=torch.float32, device="cuda")
            sg = efa.route_group(sids, E, stream=stream)
            efa.expert_dedup(self.shared_dev, x, sids, sw, sg, y=ys, accumulate=True, stream=stream)
            efa.expert_dedup(self.shared_dev, x, sids, sw, sg, y=yd, accumulate=True, stream=stream)
        torch.cuda.synchronize()
        return ys.cpu().numpy(), yd.cpu().numpy(), grp.u_and_err.cpu().numpy()

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
