"""PyTorch-facing binding of the C ABI: argument marshalling only.

PyTorch supplies device memory and the stream; every step of the expert
operation runs in the library's HIP kernels.
"""
import ctypes
from collections import namedtuple

import numpy as np
import torch

from . import _abi
from ._abi import MOE_BF16, MOE_F32, MOE_KIND_DEDUP, MOE_KIND_SLOT, check, lib

Grouping = namedtuple("Grouping", ["count", "offset", "slot_by_expert", "distinct", "u_and_err"])


def _vp(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype == torch.float32:
        return MOE_F32
    raise TypeError("weights and x must be bfloat16 or float32, got %s" % t.dtype)


def _check_dev(name, t, dtype=None, shape=None):
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))


class Layer:
    """Device weights of one MoE layer: W_gate, W_up [N][d_ff][d], W_down [N][d][d_ff],
    or, with ``packed``, W_down in the layout of ``moe_pack_w_down``,
    [N][d_ff/8][d][8] (see ``Layer.packed_copy``), or, with ``tiled``, all three in
    the tiled layout of ``moe_pack_tiled`` (same shapes, see ``Layer.tiled_copy``).
    ``shared``: the always-on experts' (W_gate, W_up, W_down), [n_shared][...] in the
    same layouts, computed in the same call as the routed experts."""

    def __init__(self, w_gate, w_up, w_down, m, packed=False, shared=None, tiled=False):
        N, d_ff, d = w_gate.shape
        _check_dev("w_gate", w_gate)
        _check_dev("w_up", w_up, w_gate.dtype, (N, d_ff, d))
        if packed and tiled:
            raise ValueError("a layer is either packed (W_down) or tiled (all three)")
        self.packed = bool(packed)
        self.tiled = bool(tiled)
        self.N, self.m, self.d, self.d_ff = N, int(m), d, d_ff
        self.dtype = w_gate.dtype
        _check_dev("w_down", w_down, w_gate.dtype, self._down_shape(N))
        self.w_gate, self.w_up, self.w_down = w_gate, w_up, w_down
        self.shared = None
        self.n_shared = 0
        ptrs = [0, 0, 0]
        if shared is not None:
            sg, su, sd = shared
            S = sg.shape[0]
            if not 1 <= S <= _abi.MOE_MAX_SHARED:
                raise ValueError("n_shared must be in 1..%d, got %d" % (_abi.MOE_MAX_SHARED, S))
            _check_dev("w_gate_shared", sg, self.dtype, (S, d_ff, d))
            _check_dev("w_up_shared", su, self.dtype, (S, d_ff, d))
            _check_dev("w_down_shared", sd, self.dtype, self._down_shape(S))
            self.shared = (sg, su, sd)
            self.n_shared = S
            ptrs = [sg.data_ptr(), su.data_ptr(), sd.data_ptr()]
        self._weights = _abi.LayerWeights(w_gate.data_ptr(), w_up.data_ptr(), w_down.data_ptr(), *ptrs)

    def _down_shape(self, E):
        return (E, self.d_ff // 8, self.d, 8) if self.packed else (E, self.d, self.d_ff)

    def desc(self, accumulate=False):
        flags = ((_abi.MOE_FLAG_ACCUMULATE if accumulate else 0) | (_abi.MOE_FLAG_WDOWN_PACKED if self.packed else 0)
                 | (_abi.MOE_FLAG_TILED if self.tiled else 0))
        return _abi.LayerDesc(self.N, self.m, self.d, self.d_ff, _dtype_code(self.w_gate), flags, self.n_shared)

    def packed_copy(self, stream=None):
        """The same layer with W_down (and the shared experts' W_down) packed by
        ``moe_pack_w_down`` (new device tensors; W_gate and W_up shared)."""
        if self.packed:
            return self
        if self.tiled:
            raise ValueError("a tiled layer cannot also be packed")

        def pk(wd):
            E = wd.shape[0]
            dst = torch.empty((E, self.d_ff // 8, self.d, 8), dtype=self.dtype, device=wd.device)
            return pack_w_down(self, wd, dst, stream=stream)
        sh = None if self.shared is None else (self.shared[0], self.shared[1], pk(self.shared[2]))
        return Layer(self.w_gate, self.w_up, pk(self.w_down), self.m, packed=True, shared=sh)

    def tiled_copy(self, stream=None):
        """The same layer with W_gate, W_up and W_down (routed and shared) copied into
        the tiled layout by ``moe_pack_tiled`` (new device tensors of the same
        shapes)."""
        if self.tiled:
            return self
        if self.packed:
            raise ValueError("tile a layer from its plain layout")

        def tl(w, mat):
            return pack_tiled(self, w, torch.empty_like(w), mat, stream=stream)
        G, D = _abi.MOE_MAT_GATE_UP, _abi.MOE_MAT_DOWN
        sh = None
        if self.shared is not None:
            sg, su, sd = self.shared
            sh = (tl(sg, G), tl(su, G), tl(sd, D))
        return Layer(tl(self.w_gate, G), tl(self.w_up, G), tl(self.w_down, D), self.m, shared=sh, tiled=True)

    def without_shared(self):
        """The routed experts alone (same tensors)."""
        return Layer(self.w_gate, self.w_up, self.w_down, self.m, packed=self.packed, tiled=self.tiled)

    @property
    def expert_bytes(self):
        return 3 * self.d * self.d_ff * self.w_gate.element_size()

    def workspace(self, n, kind=MOE_KIND_SLOT):
        """Zero-filled workspace for passes of up to n tokens (either kind)."""
        nb = max(lib().moe_workspace_bytes(ctypes.byref(self.desc()), int(n), int(k)) for k in (0, 1))
        if nb == 0:
            raise _abi.MoeError("moe_workspace_bytes", _abi.MOE_E_INVAL)
        return torch.zeros(nb, dtype=torch.uint8, device=self.w_gate.device)


def pack_w_down(layer, w_down, out, stream=None):
    """Copy W_down [E][d][d_ff] (E experts: the layer's N, or its shared experts) into
    the packed layout [E][d_ff/8][d][8] (one launch)."""
    E = w_down.shape[0]
    _check_dev("w_down", w_down, layer.dtype, (E, layer.d, layer.d_ff))
    _check_dev("out", out, layer.dtype, (E, layer.d_ff // 8, layer.d, 8))
    desc = _abi.LayerDesc(E, 1, layer.d, layer.d_ff, _dtype_code(layer.w_gate), 0, 0)
    check("moe_pack_w_down", lib().moe_pack_w_down(ctypes.byref(desc), _vp(w_down), _vp(out), _stream(stream)))
    return out


def pack_tiled(layer, w, out, mat, stream=None):
    """Copy one weight tensor of E experts (the layer's N, or its shared experts) into
    the tiled layout of ``moe_pack_tiled`` (one launch): ``mat`` MOE_MAT_GATE_UP for
    W_gate or W_up [E][d_ff][d], MOE_MAT_DOWN for W_down [E][d][d_ff]; ``out`` has the
    source's shape."""
    E = w.shape[0]
    shape = (E, layer.d_ff, layer.d) if mat == _abi.MOE_MAT_GATE_UP else (E, layer.d, layer.d_ff)
    _check_dev("w", w, layer.dtype, shape)
    _check_dev("out", out, layer.dtype, shape)
    desc = _abi.LayerDesc(E, 1, layer.d, layer.d_ff, _dtype_code(layer.w_gate), 0, 0)
    check("moe_pack_tiled", lib().moe_pack_tiled(ctypes.byref(desc), _vp(w), _vp(out), int(mat), _stream(stream)))
    return out


Routed = namedtuple("Routed", ["ids", "w", "logits", "ws"])


def router_topk(w_router, x, m, out=None, stream=None):
    """The router (``moe_router_topk``): logits [n][N] fp32, the m largest per token
    (descending, ties to the lower id) and their softmax.  Returns Routed(ids, w,
    logits, ws); pass it back as ``out`` to reuse its buffers."""
    N, d = w_router.shape
    _check_dev("w_router", w_router)
    _check_dev("x", x, w_router.dtype, (x.shape[0], d))
    n = x.shape[0]
    dev = x.device
    desc = _abi.LayerDesc(N, int(m), d, 8, _dtype_code(w_router), 0, 0)
    if out is None:
        nb = lib().moe_router_workspace_bytes(ctypes.byref(desc), n)
        if nb == 0:
            raise _abi.MoeError("moe_router_workspace_bytes", _abi.MOE_E_INVAL)
        out = Routed(torch.empty(n, m, dtype=torch.int32, device=dev), torch.empty(n, m, dtype=torch.float32, device=dev),
                     torch.empty(n, N, dtype=torch.float32, device=dev), torch.empty(nb, dtype=torch.uint8, device=dev))
    st = lib().moe_router_topk(ctypes.byref(desc), _vp(w_router), _vp(x), n, _vp(out.logits), _vp(out.ids),
                               _vp(out.w), _vp(out.ws), out.ws.numel(), _stream(stream))
    check("moe_router_topk", st)
    return out


def route_group(ids, N, out=None, stream=None):
    """Group the pass's slots by expert (one kernel launch)."""
    _check_dev("ids", ids, torch.int32)
    n, m = ids.shape
    dev = ids.device
    if out is None:
        out = Grouping(torch.empty(N, dtype=torch.int32, device=dev), torch.empty(N + 1, dtype=torch.int32, device=dev),
                       torch.empty(n * m, dtype=torch.int32, device=dev), torch.empty(N, dtype=torch.int32, device=dev),
                       torch.empty(2, dtype=torch.int32, device=dev))
    st = lib().moe_route_group(_vp(ids), n, m, N, _vp(out.count), _vp(out.offset), _vp(out.slot_by_expert),
                               _vp(out.distinct), _vp(out.u_and_err), _stream(stream))
    check("moe_route_group", st)
    return out


def _prep(layer, x, ids, w, y, ws, kind):
    n = x.shape[0]
    _check_dev("x", x, layer.dtype, (n, layer.d))
    _check_dev("ids", ids, torch.int32, (n, layer.m))
    _check_dev("w", w, torch.float32, (n, layer.m))
    if y is None:
        y = torch.empty(n, layer.d, dtype=torch.float32, device=x.device)
    _check_dev("y", y, torch.float32, (n, layer.d))
    if ws is None:
        ws = layer.workspace(n, kind)
    _check_dev("ws", ws, torch.uint8)  # its size in bytes is ws.numel()
    return n, y, ws


def _events(events):
    if events is None:
        return ctypes.c_void_p(0), 0
    arr = (ctypes.c_void_p * len(events))(*[e for e in events])
    return arr, len(events)


def _run(fn, fn_ev, layer, x, ids, w, y, ws, info, accumulate, stream, events, kind, where):
    n, y, ws = _prep(layer, x, ids, w, y, ws, kind)
    if info is not None:
        _check_dev("info", info, torch.int32, (3,))
    desc = layer.desc(accumulate)
    args = [ctypes.byref(desc), ctypes.byref(layer._weights), _vp(x), _vp(ids), _vp(w), n, _vp(y), _vp(info),
            _vp(ws), ws.numel(), _stream(stream)]
    if events is None:
        st = fn(*args)
    else:
        ev, nev = _events(events)
        st = fn_ev(*args, ev, nev)
    check(where, st)
    return y


def expert_perslot(layer, x, ids, w, y=None, ws=None, info=None, accumulate=False, stream=None, events=None):
    """The expert operation by the per-slot kernel (one launch); returns y [n][d] fp32.
    ``ws`` must come from ``layer.workspace`` (zero-filled); ``info`` an int32 [3]
    device tensor receiving (U, ids status, sync status)."""
    L = lib()
    return _run(L.moe_expert_perslot, L.moe_expert_perslot_ev, layer, x, ids, w, y, ws, info, accumulate, stream,
                events, MOE_KIND_SLOT, "moe_expert_perslot")


def expert_dedup(layer, x, ids, w, y=None, ws=None, info=None, accumulate=False, stream=None, events=None):
    """The expert operation by the deduplicating kernel (one launch; the grouping
    by expert runs inside it); returns y [n][d] fp32."""
    L = lib()
    return _run(L.moe_expert_dedup, L.moe_expert_dedup_ev, layer, x, ids, w, y, ws, info, accumulate, stream,
                events, MOE_KIND_DEDUP, "moe_expert_dedup")


def expert_auto(layer, x, ids, w, crossover, y=None, ws=None, info=None, accumulate=False, stream=None):
    """The crossover-driven switch (``moe_expert_auto``): the deduplicating kernel from
    n >= crossover tokens, the per-slot kernel below (crossover 0: always per-slot).
    Returns (y, kind run)."""
    n, y, ws = _prep(layer, x, ids, w, y, ws, MOE_KIND_DEDUP)
    if info is not None:
        _check_dev("info", info, torch.int32, (3,))
    desc = layer.desc(accumulate)
    kind = ctypes.c_int32(-1)
    st = lib().moe_expert_auto(ctypes.byref(desc), ctypes.byref(layer._weights), _vp(x), _vp(ids), _vp(w), n, _vp(y),
                               _vp(info), _vp(ws), ws.numel(), int(crossover), ctypes.byref(kind), _stream(stream))
    check("moe_expert_auto", st)
    return y, kind.value


def expert_auto_noalloc(layer, x, ids, w, crossover, y=None, info=None, accumulate=False, stream=None):
    """``moe_expert_auto_noalloc``: the same switch with no workspace argument (the
    library's per-GPU scratch array serves as workspace; nothing is allocated by the
    call itself).  Returns (y, kind run).  ``y`` should be preallocated by callers
    that cannot allocate."""
    n = x.shape[0]
    _check_dev("x", x, layer.dtype, (n, layer.d))
    _check_dev("ids", ids, torch.int32, (n, layer.m))
    _check_dev("w", w, torch.float32, (n, layer.m))
    if y is None:
        y = torch.empty(n, layer.d, dtype=torch.float32, device=x.device)
    _check_dev("y", y, torch.float32, (n, layer.d))
    if info is not None:
        _check_dev("info", info, torch.int32, (3,))
    desc = layer.desc(accumulate)
    kind = ctypes.c_int32(-1)
    st = lib().moe_expert_auto_noalloc(ctypes.byref(desc), ctypes.byref(layer._weights), _vp(x), _vp(ids), _vp(w), n,
                                       _vp(y), _vp(info), int(crossover), ctypes.byref(kind), _stream(stream))
    check("moe_expert_auto_noalloc", st)
    return y, kind.value


def kernels_per_call(kind):
    return lib().moe_kernels_per_call(int(kind))


def bytes_requested(kind, N, m, d, d_ff, dtype, ids_host):
    """Expert bytes requested by kernel ``kind`` for host ids [n][m]."""
    ids_host = np.ascontiguousarray(ids_host, dtype=np.int32)
    n = ids_host.shape[0]
    code = MOE_BF16 if dtype in ("bf16", torch.bfloat16) else MOE_F32
    desc = _abi.LayerDesc(N, m, d, d_ff, code, 0)
    v = lib().bytes_requested(int(kind), ctypes.byref(desc), ids_host.ctypes.data_as(ctypes.c_void_p), n)
    if v < 0:
        raise _abi.MoeError("bytes_requested", int(v))
    return int(v)


def step_time_model(n_max, a, m_W, E, beta, t0=0.0, D=0.0, kv=None, beta_D=1.0, phi=None, h=None):
    """Evaluate the step-time model.  E, beta, phi: [2][n_max] (kind, n-1); kv, h:
    [n_max] (k).  Returns a dict of numpy arrays trimmed to the sizes used."""
    si = _abi.StepIn()
    si.n_max, si.n_a = int(n_max), len(a)
    for i, v in enumerate(a):
        si.a[i] = float(v)
    si.m_W, si.t0, si.D, si.beta_D = float(m_W), float(t0), float(D), float(beta_D)
    kv = kv if kv is not None else [0.0] * n_max
    h = h if h is not None else [0.0] * n_max
    phi = phi if phi is not None else [[0.0] * n_max, [0.0] * n_max]
    for k in range(n_max):
        si.kv[k], si.h[k] = float(kv[k]), float(h[k])
        for p in range(2):
            si.E[p][k], si.beta[p][k], si.phi[p][k] = float(E[p][k]), float(beta[p][k]), float(phi[p][k])
    so = _abi.StepOut()
    check("step_time_model", lib().step_time_model(ctypes.byref(si), ctypes.byref(so)))
    na = len(a)
    arr = lambda c, *shape: np.ctypeslib.as_array(c).reshape(*shape) if shape else np.ctypeslib.as_array(c)  # noqa
    return {
        "tau": np.array(so.tau)[:, :n_max].copy(),
        "S": np.array(so.S)[:n_max].copy(),
        "crossover": int(so.crossover),
        "V": np.array(so.V)[:, :n_max].copy(),
        "a0": np.array(so.a0).copy(),
        "kstar": np.array(so.kstar)[:, :na].copy(),
        "speedup": np.array(so.speedup)[:, :na].copy(),
        "step_point": np.array(so.step_point)[:, :n_max].copy(),
        "convex": np.array(so.convex).copy(),
        "a1_convex": np.array(so.a1_convex).copy(),
        "rho_star": np.array(so.rho_star)[:na, :n_max].copy(),
        "rho_star_bytes": np.array(so.rho_star_bytes)[:na, :n_max].copy(),
    }


def fit_times(kind, n, U, m, t, b):
    """Least-squares fit of a kernel's times over passes with chosen ids
    (``moe_fit_times``): per-slot (t_op, c_u, c_re), deduplicating (t_op, c_g, c_t)."""
    n = np.ascontiguousarray(n, dtype=np.int32)
    U = np.ascontiguousarray(U, dtype=np.int32)
    t = np.ascontiguousarray(t, dtype=np.float64)
    if not (n.shape == U.shape == t.shape and n.ndim == 1):
        raise ValueError("n, U and t must be 1-d arrays of one length")
    coef = np.zeros(3, np.float64)
    pi32, pd = ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_double)
    st = lib().moe_fit_times(int(kind), int(n.size), n.ctypes.data_as(pi32), U.ctypes.data_as(pi32), int(m),
                             t.ctypes.data_as(pd), float(b), coef.ctypes.data_as(pd))
    check("moe_fit_times", st)
    return tuple(float(c) for c in coef)


def error_bounds(eps):
    """Factors of the Table 2 bounds for a relative bandwidth error eps (``moe_error_bounds``)."""
    out = np.zeros(5, np.float64)
    check("moe_error_bounds", lib().moe_error_bounds(float(eps), out.ctypes.data_as(ctypes.POINTER(ctypes.c_double))))
    return {"time_factor": float(out[0]), "faster_margin": float(out[1]), "delta": float(out[2]),
            "regret_factor": float(out[3]), "speedup_factor": float(out[4])}


def expert_bitmaps(ids, N):
    """Per node and layer the bitmap of its experts: ids int [V+1][L][m] -> uint64
    [V+1][L][ceil(N/64)] (argument marshalling for ``tree_select``)."""
    ids = np.asarray(ids, dtype=np.int64)
    W = (int(N) + 63) // 64
    out = np.zeros(ids.shape[:2] + (W,), np.uint64)
    for v in range(ids.shape[0]):
        for l in range(ids.shape[1]):
            for e in ids[v, l]:
                out[v, l, e // 64] |= np.uint64(1) << np.uint64(e % 64)
    return out


def tree_select(parent, p, bitmaps, K, b, beta, max_level=0, level=None):
    """The verification subtree with the largest reward over predicted cycle time
    (``moe_tree_select``).  Returns a dict: ids (sorted node ids), R, T, F, visited."""
    parent = np.ascontiguousarray(parent, dtype=np.int32)
    p = np.ascontiguousarray(p, dtype=np.float64)
    bm = np.ascontiguousarray(bitmaps, dtype=np.uint64)
    b = np.ascontiguousarray(b, dtype=np.float64)
    V = parent.size - 1
    if bm.ndim != 3 or bm.shape[0] != V + 1 or p.size != V + 1 or b.size != int(K) + 1:
        raise ValueError("shapes: parent/p [V+1], bitmaps [V+1][L][words], b [K+1]")
    lv = None if level is None else np.ascontiguousarray(level, dtype=np.int32)
    ti = _abi.TreeIn(V, bm.shape[1], bm.shape[2], int(K), parent.ctypes.data, p.ctypes.data, bm.ctypes.data,
                     b.ctypes.data, float(beta), int(max_level), None if lv is None else lv.ctypes.data)
    to = _abi.TreeOut()
    check("moe_tree_select", lib().moe_tree_select(ctypes.byref(ti), ctypes.byref(to)))
    ids = [v + 1 for v in range(64) if (to.selected >> v) & 1]
    return {"ids": ids, "R": to.R, "T": to.T, "F": to.F, "visited": to.visited}
