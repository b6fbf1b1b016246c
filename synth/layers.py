"""Shapes of the synthetic MoE layers and their seeded weights and activations.

Layer shapes (experts N, experts per token m, d_model, expert d_ff, dtype):

* ``tiny``      N=8,   m=2, d=64,   d_ff=128,   fp32 (correctness only)
* ``dsv2lite``  N=64,  m=6, d=2048, d_ff=1408,  bf16, plus 2 always-on shared experts
* ``qwen3``     N=128, m=8, d=2048, d_ff=768,   bf16, 48 such layers per pass
* ``mixtral``   N=8,   m=2, d=4096, d_ff=14336, bf16
* ``tree``      the qwen3 layer verified over a 32-node draft tree

Weights ~ N(0, 0.02^2) (0.02 read as the standard deviation), x ~ N(0, 1).
Layouts (row-major, contiguous):  W_gate, W_up [N][d_ff][d];  W_down [N][d][d_ff].
"""
from dataclasses import dataclass

import numpy as np

from . import lib

TAG_GATE, TAG_UP, TAG_DOWN, TAG_X = 1, 2, 3, 4
TAG_SHARED = 16  # shared expert s uses tags TAG_SHARED + 4*s + {1,2,3}
TAG_ROUTER = 15


@dataclass(frozen=True)
class LayerSpec:
    name: str
    N: int
    m: int
    d: int
    d_ff: int
    dtype: str          # "bf16" or "f32": weights and x
    n_shared: int = 0
    layers: int = 1
    sigma: float = 0.02

    @property
    def elem_bytes(self):
        return 2 if self.dtype == "bf16" else 4

    @property
    def expert_bytes(self):
        """Bytes of one expert's gate, up and down matrices: w = 3 d d_ff sizeof(W)."""
        return 3 * self.d * self.d_ff * self.elem_bytes


CONFIGS = {
    "tiny": LayerSpec("tiny", N=8, m=2, d=64, d_ff=128, dtype="f32"),
    "dsv2lite": LayerSpec("dsv2lite", N=64, m=6, d=2048, d_ff=1408, dtype="bf16", n_shared=2),
    "qwen3": LayerSpec("qwen3", N=128, m=8, d=2048, d_ff=768, dtype="bf16", layers=48),
    "mixtral": LayerSpec("mixtral", N=8, m=2, d=4096, d_ff=14336, dtype="bf16"),
    "tree": LayerSpec("tree", N=128, m=8, d=2048, d_ff=768, dtype="bf16"),
}


def layer_spec(name, **over):
    s = CONFIGS[name]
    if over:
        d = dict(s.__dict__)
        d.update(over)
        s = LayerSpec(**d)
    return s


def _keys(seed, layer, tag, experts):
    return [lib.key_of(seed, layer, tag, int(e)) for e in experts]


def expert_weights(spec, seed, layer, e, shared=False):
    """(W_gate[e] [d_ff][d], W_up[e] [d_ff][d], W_down[e] [d][d_ff]) of one expert."""
    base = TAG_SHARED + 4 * int(e) if shared else 0
    ee = 0 if shared else int(e)
    g = lib.blocks(_keys(seed, layer, base + TAG_GATE, [ee]), spec.d_ff * spec.d, spec.sigma, spec.dtype)
    u = lib.blocks(_keys(seed, layer, base + TAG_UP, [ee]), spec.d_ff * spec.d, spec.sigma, spec.dtype)
    dn = lib.blocks(_keys(seed, layer, base + TAG_DOWN, [ee]), spec.d * spec.d_ff, spec.sigma, spec.dtype)
    return (g.reshape(spec.d_ff, spec.d), u.reshape(spec.d_ff, spec.d), dn.reshape(spec.d, spec.d_ff))


def layer_weights(spec, seed, layer=0, shared=False, out=None):
    """Host arrays (W_gate, W_up, W_down) of all N routed experts (or the n_shared
    shared experts when ``shared``), shapes [E][d_ff][d], [E][d_ff][d], [E][d][d_ff].
    ``out`` may supply three preallocated contiguous arrays to fill."""
    E = spec.n_shared if shared else spec.N
    npdt = np.uint16 if spec.dtype == "bf16" else np.float32
    if out is None:
        out = (np.empty((E, spec.d_ff, spec.d), npdt), np.empty((E, spec.d_ff, spec.d), npdt),
               np.empty((E, spec.d, spec.d_ff), npdt))
    res = []
    for tag, arr in zip((TAG_GATE, TAG_UP, TAG_DOWN), out):
        if shared:
            keys = [lib.key_of(seed, layer, TAG_SHARED + 4 * s + tag, 0) for s in range(E)]
        else:
            keys = _keys(seed, layer, tag, range(E))
        lib.blocks(keys, spec.d_ff * spec.d, spec.sigma, spec.dtype, out=arr.reshape(-1))
        res.append(arr)
    return tuple(res)


def pass_x(spec, seed, layer, pass_id, n):
    """Activations x [n][d] of one pass (bf16 bit patterns or fp32)."""
    k = lib.key_of(seed, layer, TAG_X, pass_id)
    if spec.dtype == "bf16":
        return lib.normal_bf16(k, n * spec.d, 1.0).reshape(n, spec.d)
    return lib.normal_f32(k, n * spec.d, 1.0).reshape(n, spec.d)


def router_weights(spec, seed, layer=0, sigma=None):
    """Router W_r [N][d] (bf16 bit patterns or fp32), sigma * N(0, 1) per element.
    The default sigma makes the logits of N(0, 1) activations unit-variance
    (sigma = 1/sqrt(d)), so that top-m selections have realistic margins."""
    sg = (1.0 / np.sqrt(spec.d)) if sigma is None else sigma
    blk = lib.blocks([lib.key_of(seed, layer, TAG_ROUTER, 0)], spec.N * spec.d, sg, spec.dtype)
    return blk.reshape(spec.N, spec.d)
