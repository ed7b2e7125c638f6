"""ctypes view of libmoe.so (the C ABI declared in include/moe.h).

Loading fails loudly when the library has not been built: there is no
fallback path of any kind.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK = 0
MOE_EINVAL = -1
MOE_EUNSUPPORTED = -2
MOE_EHIP = -3
MOE_EWORKSPACE = -4
MOE_ECACHE = -5

WTYPE_F32 = 0
WTYPE_BF16 = 1
WTYPE_MXFP4 = 2
WTYPE_NVFP4 = 3

MODE_ROUTE = 0
MODE_DECODE = 1
MODE_PREFILL = 2

DECODE_MAX_T = 64
NOALLOC_SCRATCH_BYTES = 8 << 20
PLAN_MAX = 256

# every symbol include/moe.h declares
EXPORTS = (
    "moe_expert_layout", "moe_workspace_bytes", "moe_route", "moe_decode",
    "moe_route_decode", "moe_route_decode_noalloc", "moe_decode_launch_tokens", "moe_prefill", "moe_merge_partials", "moe_quantize_mxfp4",
    "moe_pack_expert", "moe_decode_status", "moe_debug_prefill_layout", "moe_debug_dot_fp4", "moe_debug_dequant_mxfp4", "moe_debug_mfma_fp4_tile", "moe_debug_read_probe", "moe_debug_wave_scan", "moe_qstar",
    "moe_planner_create", "moe_planner_destroy", "moe_planner_set_bandwidths",
    "moe_planner_plan", "moe_planner_rollback", "moe_planner_slot_table",
    "moe_planner_resize", "moe_planner_n_slots", "moe_cache_resize",
    "moe_layer_stream_create", "moe_layer_stream_destroy", "moe_layer_stream_acquire",
    "moe_layer_stream_release",
    "moe_cache_create", "moe_cache_destroy", "moe_cache_set_bandwidths",
    "moe_cache_plan", "cache_fill", "moe_cache_release",
    "moe_cache_debug_fail_fills", "moe_cache_planner", "moe_probe_bandwidths",
    "moe_host_experts", "moe_host_expert_rate", "moe_last_error", "moe_abi_version",
)


class MoeDesc(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("has_shared", ctypes.c_int32), ("renorm_topk", ctypes.c_int32),
                ("wtype", ctypes.c_int32), ("router_wtype", ctypes.c_int32)]


_I32xP = ctypes.c_int32 * PLAN_MAX


class MoePlan(ctypes.Structure):
    _fields_ = [("layer", ctypes.c_int32), ("n_selected", ctypes.c_int32),
                ("n_hits", ctypes.c_int32), ("n_misses", ctypes.c_int32),
                ("q", ctypes.c_int32), ("n_host", ctypes.c_int32),
                ("selected", _I32xP), ("hits", _I32xP), ("misses", _I32xP),
                ("fill_expert", _I32xP), ("fill_slot", _I32xP),
                ("victim_layer", _I32xP), ("victim_expert", _I32xP),
                ("host_expert", _I32xP), ("hit_slot", _I32xP)]


class MoeError(RuntimeError):
    def __init__(self, status, what):
        super().__init__(f"{what} (status {status})")
        self.status = status


_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m sparse_expert_execution_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ, D = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                          ctypes.c_size_t, ctypes.c_double)
    DP = ctypes.POINTER(MoeDesc)
    PP = ctypes.POINTER(MoePlan)
    sig = {
        "moe_expert_layout": (ctypes.c_int, [DP, ctypes.POINTER(SZ), ctypes.POINTER(SZ)]),
        "moe_workspace_bytes": (SZ, [DP, I32, I32]),
        "moe_route": (ctypes.c_int, [DP, P, P, I32, P, P, P, SZ, P]),
        "moe_decode": (ctypes.c_int, [DP, P, I32, P, P, P, P, P, P, P, SZ, P]),
        "moe_prefill": (ctypes.c_int, [DP, P, I32, P, P, P, P, P, P, P, SZ, P]),
        "moe_route_decode": (ctypes.c_int, [DP, P, P, I32, P, P, P, P, P, P, P, SZ, P]),
        "moe_route_decode_noalloc": (ctypes.c_int, [DP, P, P, I32, P, P, P, P, P, P, P, P]),
        "moe_decode_launch_tokens": (I32, [DP]),
        "moe_merge_partials": (ctypes.c_int, [P, P, P, SZ, P]),
        "moe_quantize_mxfp4": (ctypes.c_int, [P, I32, I32, I64, P, P, P]),
        "moe_pack_expert": (ctypes.c_int, [DP, P, P, P, I32, P, P]),
        "moe_debug_dequant_mxfp4": (ctypes.c_int, [P, P, I64, P, P]),
        "moe_debug_dot_fp4": (ctypes.c_int, [I32, P, P, P, I64, I32, P, P]),
        "moe_decode_status": (ctypes.c_int, [P, SZ, P, I32, P]),
        "moe_debug_prefill_layout": (ctypes.c_int, [DP, I32, ctypes.POINTER(I64)]),
        "moe_debug_mfma_fp4_tile": (ctypes.c_int, [P, P, P, P, P, P]),
        "moe_debug_read_probe": (ctypes.c_int, [P, SZ, I32, P, P]),
        "moe_debug_wave_scan": (ctypes.c_int, [P, P, I32, P]),
        "moe_qstar": (I32, [I32, D, D]),
        "moe_planner_create": (ctypes.c_int, [ctypes.POINTER(P), I32, I32, I32]),
        "moe_planner_destroy": (None, [P]),
        "moe_planner_set_bandwidths": (ctypes.c_int, [P, D, D]),
        "moe_planner_plan": (ctypes.c_int, [P, I32, P, P, I32, I32, PP]),
        "moe_planner_rollback": (ctypes.c_int, [P]),
        "moe_planner_slot_table": (ctypes.c_int, [P, I32, P]),
        "moe_planner_resize": (ctypes.c_int, [P, I32, P]),
        "moe_planner_n_slots": (ctypes.c_int32, [P]),
        "moe_cache_resize": (ctypes.c_int, [P, P, I32, P]),
        "moe_layer_stream_create": (ctypes.c_int, [ctypes.POINTER(P), P, I32, SZ, P, P]),
        "moe_layer_stream_destroy": (None, [P]),
        "moe_layer_stream_acquire": (ctypes.c_int, [P, I32, P, P, ctypes.POINTER(P)]),
        "moe_layer_stream_release": (ctypes.c_int, [P, I32, P]),
        "moe_cache_create": (ctypes.c_int, [ctypes.POINTER(P), P, I32, I32, SZ, P, I32, P]),
        "moe_cache_destroy": (None, [P]),
        "moe_cache_set_bandwidths": (ctypes.c_int, [P, D, D]),
        "moe_cache_plan": (ctypes.c_int, [P, I32, P, P, I32, I32, PP]),
        "cache_fill": (ctypes.c_int, [P, PP, P, P]),
        "moe_cache_release": (ctypes.c_int, [P, PP, P]),
        "moe_cache_debug_fail_fills": (ctypes.c_int, [P, I32]),
        "moe_cache_planner": (P, [P]),
        "moe_probe_bandwidths": (ctypes.c_int, [P, P, SZ, I32, I32, P,
                                                ctypes.POINTER(D), ctypes.POINTER(D)]),
        "moe_host_experts": (ctypes.c_int, [P, P, I32, P, P, P, P, P, P, I32]),
        "moe_host_expert_rate": (ctypes.c_int, [P, P, I32, I32, I32, ctypes.POINTER(D)]),
        "moe_last_error": (ctypes.c_char_p, []),
        "moe_abi_version": (I32, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def check(status, what):
    if status != MOE_OK:
        msg = lib().moe_last_error().decode(errors="replace")
        raise MoeError(status, f"{what}: {msg}")
    return status
