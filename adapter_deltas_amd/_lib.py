"""ctypes prototypes of include/lora.h.  Loading fails loudly if liblora.so is
missing: there is no fallback path."""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblora.so")

LORA_OK = 0
STATUS = {
    0: "LORA_OK", -1: "LORA_ERR_ARG", -2: "LORA_ERR_SHAPE", -3: "LORA_ERR_DTYPE",
    -4: "LORA_ERR_RANK", -5: "LORA_ERR_CAPACITY", -6: "LORA_ERR_UNKNOWN_ADAPTER",
    -7: "LORA_ERR_SLOT", -8: "LORA_ERR_MISMATCH", -9: "LORA_ERR_HIP",
}
DTYPE = {"bf16": 1, "fp16": 2, "fp32": 3}
MAX_SLICES = 4
MAX_RANK = 256
DECODE_SEG_ROWS = 8
SEG_WORDS = 16
GATHER_MIN_RANK = 128         # LORA_GATHER_MIN_RANK
DEVICE_ROUTING_MAX_TOKENS = 8192   # LORA_DEVICE_ROUTING_MAX_TOKENS
PREFILL_SEG_ROWS = 64
NOALLOC_SCRATCH_BYTES = 8388608   # LORA_NOALLOC_SCRATCH_BYTES

# every symbol include/lora.h declares
EXPORTS = (
    "lora_last_error", "lora_version",
    "lora_pool_bytes", "lora_pool_create", "lora_pool_destroy", "lora_pool_load",
    "lora_pool_unload", "lora_pool_slot_of",
    "lora_routing_bytes", "lora_routing_create", "lora_routing_destroy",
    "lora_build_routing", "lora_routing_get_info", "lora_plan_routing",
    "lora_pool_load_folded",
    "lora_build_routing_rows", "lora_plan_rows",
    "lora_routing_token_slots", "lora_build_routing_device", "lora_build_routing_moe",
    "lora_routing_device_counts",
    "lora_shrink", "lora_expand", "lora_workspace_bytes", "lora_delta_apply",
    "lora_delta_apply_noalloc",
    "lora_linear_workspace_bytes", "lora_linear_delta",
)


class LaneDesc(ctypes.Structure):
    _fields_ = [
        ("h_in", ctypes.c_int32),
        ("n_slices", ctypes.c_int32),
        ("h_out", ctypes.c_int32 * MAX_SLICES),
        ("max_slots", ctypes.c_int32),
        ("max_rank", ctypes.c_int32),
        ("x_dtype", ctypes.c_int32),
    ]


class RoutingInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_tokens", "n_active", "n_segments", "n_decode_segments",
        "n_prefill_segments", "n_distinct", "n_admitted_seqs", "n_seqs",
        "n_gather_segments")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build the HIP library first "
            "(python -c 'import __graft_entry__; __graft_entry__.build()')")
    lib = ctypes.CDLL(path)
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    PI32, PI64 = ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)
    PP = ctypes.POINTER(ctypes.c_void_p)
    sig = {
        "lora_last_error": (ctypes.c_char_p, []),
        "lora_version": (ctypes.c_char_p, []),
        "lora_pool_bytes": (I32, [ctypes.POINTER(LaneDesc), PI64]),
        "lora_pool_create": (I32, [ctypes.POINTER(LaneDesc), P, I64, P, PP]),
        "lora_pool_destroy": (I32, [P]),
        "lora_pool_load": (I32, [P, I32, I32, PP, PI64, I64, PP, PI64, PI32,
                                 ctypes.POINTER(ctypes.c_float), I32, P, PI32]),
        "lora_pool_load_folded": (I32, [P, I32, I32, PP, PI64, I64, PP, PI64, PI32,
                                        ctypes.POINTER(ctypes.c_float), P, I64, P, PI32]),
        "lora_pool_unload": (I32, [P, I32]),
        "lora_pool_slot_of": (I32, [P, I32, PI32]),
        "lora_routing_bytes": (I32, [I32, PI64]),
        "lora_routing_create": (I32, [I32, I32, P, I64, PP]),
        "lora_routing_destroy": (I32, [P]),
        "lora_build_routing": (I32, [P, I32, PI32, PI32, I32, I32, P,
                                     ctypes.POINTER(ctypes.c_uint8), PI32, P]),
        "lora_routing_get_info": (I32, [P, ctypes.POINTER(RoutingInfo)]),
        "lora_plan_routing": (I32, [I32, PI32, PI32, I32, I32, I32, PI32, PI32, PI32, I32, I32,
                                    PI32, I64, PI32, ctypes.POINTER(RoutingInfo),
                                    ctypes.POINTER(ctypes.c_uint8)]),
        "lora_routing_token_slots": (I32, [P, PP]),
        "lora_build_routing_device": (I32, [P, P, I32, P, P]),
        "lora_build_routing_moe": (I32, [P, P, I32, P, P, I32, I32, P, P]),
        "lora_build_routing_rows": (I32, [P, I32, PI32, ctypes.POINTER(ctypes.c_uint8), P, P]),
        "lora_plan_rows": (I32, [I32, PI32, ctypes.POINTER(ctypes.c_uint8), I32, PI32, PI32, I64,
                                 PI32, ctypes.POINTER(RoutingInfo)]),
        "lora_routing_device_counts": (I32, [P, PP]),
        "lora_shrink": (I32, [P, P, P, I64, P, P]),
        "lora_expand": (I32, [P, P, P, P, I64, P]),
        "lora_workspace_bytes": (I32, [P, P, PI64]),
        "lora_delta_apply": (I32, [P, P, P, I64, P, I64, P, I64, P]),
        "lora_delta_apply_noalloc": (I32, [P, P, P, I64, P, I64, P]),
        "lora_linear_workspace_bytes": (I32, [P, P, PI64]),
        "lora_linear_delta": (I32, [P, P, I32, P, I64, P, I64, P, I64, P, I64, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib
