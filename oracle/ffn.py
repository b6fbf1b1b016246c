"""ctypes wrapper of ``moe_oracle.c`` (test infrastructure only).

Composition of a pass (Lan, arXiv:2610.34440, Section 1; the DeepSeek-V2-Lite
shape adds always-on shared experts with routing weight 1, Section 4.4):
    y_t = fp32( sum_j w_tj FFN_{e_tj}(x_t) + sum_s FFN_shared_s(x_t) )
with every term and sum in double and a single rounding to fp32.
"""
import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")
_LOCK = threading.Lock()
_LIB = None

OR_OK, OR_E_INVAL, OR_E_DTYPE, OR_E_IDS = 0, -1, -2, -5
_DT = {"f32": 0, "bf16": 1}


def build(force=False):
    """Compile liboracle.so: gcc -O2, no fast-math, single thread."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fno-fast-math", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


def _configure(L):
    i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    L.oracle_route_group.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, vp]
    L.oracle_route_group.restype = ctypes.c_int
    L.oracle_union_count.argtypes = [vp, i32, i32, i32]
    L.oracle_union_count.restype = i32
    L.oracle_union_count_batch.argtypes = [vp, i64, i32, i32, i32, vp]
    L.oracle_bytes.argtypes = [i32, i32, i32, i32, i32, i32, vp, i32]
    L.oracle_bytes.restype = i64
    L.oracle_expert_apply.argtypes = [i32, i32, i32, vp, vp, vp, i32, vp, vp]
    L.oracle_expert_apply.restype = ctypes.c_int
    L.oracle_moe_ffn.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, i32, vp, vp, vp, i32, vp]
    L.oracle_moe_ffn.restype = ctypes.c_int
    return L


def _lib():
    global _LIB
    with _LOCK:
        if _LIB is None:
            if not os.path.exists(_SO):
                build()
            _LIB = _configure(ctypes.CDLL(_SO))
    return _LIB


class use_library:
    """Context manager that points this module at another build of the oracle
    source (used by the tests that plant mistakes in a copy of it)."""

    def __init__(self, path):
        self.path = path

    def __enter__(self):
        global _LIB
        _lib()
        self._saved = _LIB
        _LIB = _configure(ctypes.CDLL(self.path))
        return self

    def __exit__(self, *exc):
        global _LIB
        _LIB = self._saved
        return False


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def route_group(ids, N):
    """Returns (status, count[N], offset[N+1], slot_by_expert[nm], distinct[N], U)."""
    ids = _c(ids, np.int32)
    n, m = ids.shape
    count = np.empty(N, np.int32)
    offset = np.empty(N + 1, np.int32)
    sbe = np.empty(n * m, np.int32)
    distinct = np.empty(N, np.int32)
    U = np.zeros(1, np.int32)
    st = _lib().oracle_route_group(ids.ctypes.data, n, m, N, count.ctypes.data, offset.ctypes.data,
                                   sbe.ctypes.data, distinct.ctypes.data, U.ctypes.data)
    return st, count, offset, sbe, distinct, int(U[0])


def union_count(ids, N):
    ids = _c(ids, np.int32)
    n, m = ids.shape
    return int(_lib().oracle_union_count(ids.ctypes.data, n, m, N))


def union_count_batch(ids, N):
    """ids [B][n][m] -> X(n) of each pass."""
    ids = _c(ids, np.int32)
    B, n, m = ids.shape
    out = np.empty(B, np.int32)
    _lib().oracle_union_count_batch(ids.ctypes.data, B, n, m, N, out.ctypes.data)
    return out


def bytes_requested(kind, N, m, d, d_ff, elem_bytes, ids):
    ids = _c(ids, np.int32)
    n = ids.shape[0]
    return int(_lib().oracle_bytes(kind, N, m, d, d_ff, elem_bytes, ids.ctypes.data, n))


def expert_apply(wg, wu, wd, x, dtype, xdtype=None):
    """One expert on one token, double result o [d]."""
    xdtype = xdtype or dtype
    npw = np.uint16 if dtype == "bf16" else np.float32
    npx = np.uint16 if xdtype == "bf16" else np.float32
    wg, wu, wd, x = _c(wg, npw), _c(wu, npw), _c(wd, npw), _c(x, npx)
    d_ff, d = wg.shape
    assert wu.shape == (d_ff, d) and wd.shape == (d, d_ff) and x.shape == (d,)
    o = np.empty(d, np.float64)
    st = _lib().oracle_expert_apply(d, d_ff, _DT[dtype], wg.ctypes.data, wu.ctypes.data, wd.ctypes.data,
                                    _DT[xdtype], x.ctypes.data, o.ctypes.data)
    if st != OR_OK:
        raise ValueError("oracle_expert_apply status %d" % st)
    return o


def moe_ffn_f64(Wg, Wu, Wd, x, ids, w, dtype, xdtype=None, acc=None):
    """acc [n][d] (double) += sum_j w_tj FFN_{e_tj}(x_t).  Raises on invalid ids."""
    xdtype = xdtype or dtype
    npw = np.uint16 if dtype == "bf16" else np.float32
    npx = np.uint16 if xdtype == "bf16" else np.float32
    Wg, Wu, Wd, x = _c(Wg, npw), _c(Wu, npw), _c(Wd, npw), _c(x, npx)
    ids, w = _c(ids, np.int32), _c(w, np.float32)
    N, d_ff, d = Wg.shape
    n, m = ids.shape
    assert Wu.shape == (N, d_ff, d) and Wd.shape == (N, d, d_ff) and x.shape == (n, d)
    if acc is None:
        acc = np.zeros((n, d), np.float64)
    assert acc.dtype == np.float64 and acc.shape == (n, d) and acc.flags.c_contiguous
    st = _lib().oracle_moe_ffn(N, m, d, d_ff, _DT[dtype], Wg.ctypes.data, Wu.ctypes.data, Wd.ctypes.data,
                               _DT[xdtype], x.ctypes.data, ids.ctypes.data, w.ctypes.data, n, acc.ctypes.data)
    if st != OR_OK:
        raise ValueError("oracle_moe_ffn status %d" % st)
    return acc


def moe_ffn(Wg, Wu, Wd, x, ids, w, dtype, shared=None):
    """fp32 y [n][d] of a pass; ``shared`` = (Sg, Su, Sd) always-on experts, weight 1."""
    acc = moe_ffn_f64(Wg, Wu, Wd, x, ids, w, dtype)
    if shared is not None:
        Sg, Su, Sd = shared
        E = Sg.shape[0]
        n = x.shape[0]
        sids = np.tile(np.arange(E, dtype=np.int32), (n, 1))
        sw = np.ones((n, E), np.float32)
        moe_ffn_f64(Sg, Su, Sd, x, sids, sw, dtype, acc=acc)
    return acc.astype(np.float32)
