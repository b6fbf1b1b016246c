"""MoE expert operation of a speculative-decoding verification pass on MI355X.

Per-slot and deduplicating expert kernels (hand-written HIP for gfx950) behind the
C ABI of ``include/moe_expert.h``, plus the host byte accounting and step-time
model.  This package is the thin Python binding; it fails loudly when the native
library is missing.
"""
from ._abi import (  # noqa: F401
    MOE_KIND_DEDUP, MOE_KIND_SLOT, MOE_MAT_DOWN, MOE_MAT_GATE_UP, MoeError, lib,
)
from .ops import (  # noqa: F401
    Grouping, Layer, bytes_requested, error_bounds, expert_auto, expert_auto_noalloc, expert_bitmaps, expert_dedup,
    expert_perslot, fit_times, kernels_per_call, pack_tiled, pack_w_down, route_group, router_topk, step_time_model,
    tree_select,
)
