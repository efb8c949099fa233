"""ctypes binding of libmoe_w4a16.so (argument marshalling only).

Every function here forwards to the C entry point of the same name in
include/moe_w4a16.h.  Tensors are passed by their data pointers; streams are
hipStream_t handles (``torch.cuda.current_stream().cuda_stream``).  Nothing in
this module computes any part of the layer.
"""
from __future__ import annotations

import ctypes as C
import os

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_w4a16.so")

MOE_OK, MOE_E_ARG, MOE_E_SHAPE, MOE_E_OOM, MOE_E_HIP, MOE_E_CAPACITY = 0, 1, 2, 3, 4, 5
MOE_E_NOT_REGISTERED, MOE_E_TRANSFER, MOE_E_FAULTED, MOE_E_DEVICE = 6, 7, 8, 9
STATUS_NAMES = {0: "MOE_OK", 1: "MOE_E_ARG", 2: "MOE_E_SHAPE", 3: "MOE_E_OOM", 4: "MOE_E_HIP",
                5: "MOE_E_CAPACITY", 6: "MOE_E_NOT_REGISTERED", 7: "MOE_E_TRANSFER",
                8: "MOE_E_FAULTED", 9: "MOE_E_DEVICE"}

MOE_RESIDENT_ALL, MOE_POLICY_LRU, MOE_POLICY_LFU, MOE_POLICY_LRU_FREQ = 0, 1, 2, 3
MOE_FLAG_ROUTER_EXACT_ALWAYS = 1
MOE_FLAG_FORCE_GEMV = 2
MOE_FLAG_FORCE_MFMA = 4
MOE_FLAG_NO_FUSED = 8
MOE_FLAG_STAGED_TRANSPORT = 16
MOE_FLAG_GUESS_AHEAD = 32
MOE_FLAG_TEST_GUESS_LOWEST = 64
MOE_FLAG_TEST_GUESS_SHIFTED = 128
MOE_FLAG_TEST_GUESS_NONE = 256
MOE_MAX_COPY_DELAY_US = 100000


class moe_config(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("n_experts", C.c_int32), ("inter", C.c_int32),
                ("top_k", C.c_int32), ("renorm", C.c_int32), ("n_layers", C.c_int32),
                ("shared_inter", C.c_int32), ("group", C.c_int32), ("max_tokens", C.c_int32),
                ("device", C.c_int32), ("policy", C.c_int32), ("slots_per_layer", C.c_int32),
                ("flags", C.c_uint32), ("staging_blobs", C.c_int32), ("spare_rows", C.c_int32)]


class moe_cache_counters(C.Structure):
    _fields_ = [("accesses", C.c_uint64), ("hits", C.c_uint64), ("misses", C.c_uint64),
                ("evictions", C.c_uint64), ("h2d_bytes", C.c_uint64), ("d2h_bytes", C.c_uint64),
                ("failures", C.c_uint64), ("h2d_seconds", C.c_double),
                ("prefetches", C.c_uint64), ("prefetch_used", C.c_uint64), ("pinned", C.c_uint64)]


class moe_skew_report(C.Structure):
    _fields_ = [("top10", C.c_double), ("top20", C.c_double), ("top30", C.c_double),
                ("entropy_bits", C.c_double), ("distinct", C.c_int32), ("selections", C.c_int64)]


class moe_cache_event(C.Structure):
    _fields_ = [("step", C.c_int32), ("layer", C.c_int32), ("expert", C.c_int32),
                ("hit", C.c_int32), ("slot", C.c_int32), ("victim", C.c_int32)]

    def as_tuple(self):
        return (self.step, self.layer, self.expert, self.hit, self.slot, self.victim)


_P = C.c_void_p
_I = C.c_int32
# name: (restype, argtypes) -- mirrors include/moe_w4a16.h
SIGNATURES = {
    "moe_create": (_I, [C.POINTER(moe_config), C.POINTER(_P)]),
    "moe_destroy": (None, [_P]),
    "moe_last_error": (C.c_char_p, [_P]),
    "moe_register_layer": (_I, [_P, _I, _P, _P, _P, _P, _P]),
    "moe_route": (_I, [_P, _I, _P, _I, _P, _P, _P, _P, _P]),
    "moe_expert_forward": (_I, [_P, _I, _P, _I, _P, _P, _P, _P]),
    "moe_expert_forward_noalloc": (_I, [_P, _I, _P, _I, _P, _P, _P, _P]),
    "moe_stack_forward": (_I, [_P, _I, _I, _P, _I, _P, _P, _P, _P, _P]),
    "moe_stack_forward_into": (_I, [_P, _I, _I, _P, _P, _I, _P, _P, _P, _P, _P]),
    "moe_check_device_errors": (_I, [_P, _P, C.POINTER(C.c_uint32)]),
    "moe_cache_ensure": (_I, [_P, _I, _P, _I, _P, _I, _P]),
    "moe_cache_prefetch": (_I, [_P, _I, _P, _I, _I, _P]),
    "moe_cache_pin": (_I, [_P, _I, _P, _I, _I, _P]),
    "moe_rmsnorm": (_I, [_P, _P, _I, _P, _P]),
    "moe_stack_forward_pooled": (_I, [_P, _I, _I, _P, _I, _I, _I, _P, _P, _P]),
    "moe_cache_stats": (_I, [_P, _I, C.POINTER(moe_cache_counters)]),
    "moe_cache_event_log": (_I, [_P, _I, C.POINTER(moe_cache_event), _I, C.POINTER(_I)]),
    "moe_debug_inject_transfer_failure": (_I, [_P, _I, _I]),
    "moe_debug_delay_copies": (_I, [_P, _I]),
    "moe_timer_enable": (_I, [_P, _I]),
    "moe_timer_read": (_I, [_P, C.POINTER(C.c_double), C.POINTER(C.c_int64)]),
    "moe_fused_phase_stamps": (_I, [_P, _P, C.c_int64, C.POINTER(_I), C.POINTER(_I), C.POINTER(_I)]),
    "moe_policy_new": (_P, [_I, _I, _I, _I]),
    "moe_policy_free": (None, [_P]),
    "moe_policy_access": (_I, [_P, _P, _I, _I, _P]),
    "moe_policy_prefetch": (_I, [_P, _P, _I, _I]),
    "moe_policy_pin": (_I, [_P, _P, _I, _I]),
    "moe_trace_policy_pinned": (_I, [_I, _P, _I, _I, _I, _I, _P, _I, C.POINTER(C.c_int64), C.POINTER(C.c_int64)]),
    "moe_policy_event_count": (_I, [_P]),
    "moe_policy_events": (_I, [_P, C.POINTER(moe_cache_event), _I]),
    "moe_trace_opt": (_I, [_P, _I, _I, _I, _I, C.POINTER(C.c_int64), C.POINTER(C.c_int64)]),
    "moe_trace_policy": (_I, [_I, _P, _I, _I, _I, _I, C.POINTER(C.c_int64), C.POINTER(C.c_int64)]),
    "moe_trace_top_share": (_I, [_P, _I, _I, _I, _I, C.POINTER(C.c_double)]),
    "moe_trace_skew": (_I, [_P, _I, _I, _I, C.POINTER(moe_skew_report)]),
}

_lib = None


def lib_path() -> str:
    return _LIB_PATH


def load() -> C.CDLL:
    """Load the HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(
                f"{_LIB_PATH} is missing: build it with "
                "`python w4a16_routed_expert_router_amd/build_lib.py`")
        lib = C.CDLL(_LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class MoEError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


def check(status: int, ctx=None) -> None:
    if status != MOE_OK:
        msg = load().moe_last_error(ctx)
        raise MoEError(status, msg.decode() if msg else "")


def ptr(t) -> int | None:
    """Data pointer of a tensor / numpy array, or None."""
    if t is None:
        return None
    if hasattr(t, "data_ptr"):
        return t.data_ptr()
    return t.ctypes.data
