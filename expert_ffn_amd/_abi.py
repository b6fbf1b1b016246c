"""ctypes declarations of ``include/moe_expert.h`` (argument marshalling only).

Loading fails loudly when ``libmoe_expert.so`` has not been built: there is no
fallback path.
"""
import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
SO_PATH = os.path.join(HERE, "libmoe_expert.so")

MOE_OK, MOE_E_INVAL, MOE_E_DTYPE, MOE_E_WORKSPACE, MOE_E_HIP, MOE_E_IDS = 0, -1, -2, -3, -4, -5
MOE_F32, MOE_BF16 = 0, 1
MOE_KIND_SLOT, MOE_KIND_DEDUP = 0, 1
MOE_MAX_SLOTS, MOE_MAX_TOKENS, MOE_MAX_EXPERTS, MOE_MAX_SHARED = 256, 64, 1024, 16
MOE_FLAG_ACCUMULATE = 1
MOE_FLAG_WDOWN_PACKED = 2
MOE_FLAG_TILED = 4
MOE_MAT_GATE_UP, MOE_MAT_DOWN = 0, 1
MOE_STEP_NMAX, MOE_STEP_AMAX = 16, 64
MOE_SCRATCH_BYTES = 16 << 20

STATUS_NAMES = {0: "MOE_OK", -1: "MOE_E_INVAL", -2: "MOE_E_DTYPE", -3: "MOE_E_WORKSPACE",
                -4: "MOE_E_HIP", -5: "MOE_E_IDS"}

# every symbol the header declares
EXPORTS = ("moe_route_group", "moe_workspace_bytes", "moe_expert_perslot", "moe_expert_dedup",
           "moe_kernels_per_call", "moe_expert_perslot_ev", "moe_expert_dedup_ev", "bytes_requested",
           "step_time_model", "moe_pack_w_down", "moe_fit_times", "moe_error_bounds",
           "moe_router_topk", "moe_router_workspace_bytes", "moe_tree_select",
           "moe_expert_auto", "moe_pack_tiled", "moe_expert_auto_noalloc")


class MoeError(RuntimeError):
    def __init__(self, where, status):
        super().__init__("%s failed: %s (%d)" % (where, STATUS_NAMES.get(status, "?"), status))
        self.status = status


class LayerDesc(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int32), ("m", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("d_ff", ctypes.c_int32), ("dtype", ctypes.c_int32), ("flags", ctypes.c_uint32),
                ("n_shared", ctypes.c_int32)]


class LayerWeights(ctypes.Structure):
    _fields_ = [("w_gate", ctypes.c_void_p), ("w_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p),
                ("w_gate_shared", ctypes.c_void_p), ("w_up_shared", ctypes.c_void_p),
                ("w_down_shared", ctypes.c_void_p)]


MOE_TREE_MAXV, MOE_TREE_MAXK, MOE_TREE_MAXW = 63, 16, 16


class TreeIn(ctypes.Structure):
    _fields_ = [("V", ctypes.c_int32), ("L", ctypes.c_int32), ("words", ctypes.c_int32), ("K", ctypes.c_int32),
                ("parent", ctypes.c_void_p), ("p", ctypes.c_void_p), ("bitmap", ctypes.c_void_p),
                ("b", ctypes.c_void_p), ("beta", ctypes.c_double), ("max_level", ctypes.c_int32),
                ("level", ctypes.c_void_p)]


class TreeOut(ctypes.Structure):
    _fields_ = [("selected", ctypes.c_uint64), ("count", ctypes.c_int32), ("F", ctypes.c_int32),
                ("R", ctypes.c_double), ("T", ctypes.c_double), ("visited", ctypes.c_int64)]


_NM, _AM = MOE_STEP_NMAX, MOE_STEP_AMAX
_D = ctypes.c_double
_I = ctypes.c_int32


class StepIn(ctypes.Structure):
    _fields_ = [("n_max", _I), ("n_a", _I), ("a", _D * _AM), ("m_W", _D), ("t0", _D), ("D", _D),
                ("kv", _D * _NM), ("beta_D", _D), ("E", (_D * _NM) * 2), ("beta", (_D * _NM) * 2),
                ("phi", (_D * _NM) * 2), ("h", _D * _NM)]


class StepOut(ctypes.Structure):
    _fields_ = [("tau", (_D * _NM) * 2), ("S", _D * _NM), ("crossover", _I), ("V", (_D * _NM) * 2),
                ("a0", _D * 2), ("kstar", (_I * _AM) * 2), ("speedup", (_D * _AM) * 2),
                ("step_point", (_D * _NM) * 2), ("convex", _I * 2), ("a1_convex", _D * 2),
                ("rho_star", (_D * _NM) * _AM), ("rho_star_bytes", (_D * _NM) * _AM)]


_LIB = None
_LOCK = threading.Lock()


def lib():
    """The loaded library; raises when it is missing (build with
    ``python -m expert_ffn_amd.build``)."""
    global _LIB
    with _LOCK:
        if _LIB is None:
            if not os.path.exists(SO_PATH):
                raise RuntimeError("libmoe_expert.so is not built (%s); run python -m expert_ffn_amd.build"
                                   % SO_PATH)
            L = ctypes.CDLL(SO_PATH)
            vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
            pdesc, pw = ctypes.POINTER(LayerDesc), ctypes.POINTER(LayerWeights)
            L.moe_route_group.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, vp, vp]
            L.moe_route_group.restype = ctypes.c_int
            L.moe_workspace_bytes.argtypes = [pdesc, i32, i32]
            L.moe_workspace_bytes.restype = sz
            L.moe_expert_perslot.argtypes = [pdesc, pw, vp, vp, vp, i32, vp, vp, vp, sz, vp]
            L.moe_expert_perslot.restype = ctypes.c_int
            L.moe_expert_dedup.argtypes = [pdesc, pw, vp, vp, vp, i32, vp, vp, vp, sz, vp]
            L.moe_expert_dedup.restype = ctypes.c_int
            L.moe_kernels_per_call.argtypes = [i32]
            L.moe_kernels_per_call.restype = ctypes.c_int
            L.moe_expert_perslot_ev.argtypes = [pdesc, pw, vp, vp, vp, i32, vp, vp, vp, sz, vp, vp, i32]
            L.moe_expert_perslot_ev.restype = ctypes.c_int
            L.moe_expert_dedup_ev.argtypes = [pdesc, pw, vp, vp, vp, i32, vp, vp, vp, sz, vp, vp, i32]
            L.moe_expert_dedup_ev.restype = ctypes.c_int
            L.bytes_requested.argtypes = [i32, pdesc, vp, i32]
            L.bytes_requested.restype = i64
            L.step_time_model.argtypes = [ctypes.POINTER(StepIn), ctypes.POINTER(StepOut)]
            L.step_time_model.restype = ctypes.c_int
            L.moe_pack_w_down.argtypes = [pdesc, vp, vp, vp]
            L.moe_pack_w_down.restype = ctypes.c_int
            L.moe_pack_tiled.argtypes = [pdesc, vp, vp, i32, vp]
            L.moe_pack_tiled.restype = ctypes.c_int
            pi32, pd = ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_double)
            L.moe_fit_times.argtypes = [ctypes.c_int32, ctypes.c_int32, pi32, pi32, ctypes.c_int32, pd,
                                        ctypes.c_double, pd]
            L.moe_fit_times.restype = ctypes.c_int
            L.moe_error_bounds.argtypes = [ctypes.c_double, pd]
            L.moe_error_bounds.restype = ctypes.c_int
            L.moe_router_topk.argtypes = [pdesc, vp, vp, ctypes.c_int32, vp, vp, vp, vp, sz, vp]
            L.moe_router_topk.restype = ctypes.c_int
            L.moe_router_workspace_bytes.argtypes = [pdesc, ctypes.c_int32]
            L.moe_router_workspace_bytes.restype = sz
            L.moe_tree_select.argtypes = [ctypes.POINTER(TreeIn), ctypes.POINTER(TreeOut)]
            L.moe_tree_select.restype = ctypes.c_int
            L.moe_expert_auto.argtypes = [pdesc, pw, vp, vp, vp, i32, vp, vp, vp, sz, i32, vp, vp]
            L.moe_expert_auto.restype = ctypes.c_int
            L.moe_expert_auto_noalloc.argtypes = [pdesc, pw, vp, vp, vp, i32, vp, vp, i32, vp, vp]
            L.moe_expert_auto_noalloc.restype = ctypes.c_int
            _LIB = L
    return _LIB


def check(where, status):
    if status != MOE_OK:
        raise MoeError(where, status)
