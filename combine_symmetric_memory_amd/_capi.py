"""ctypes declarations of include/cco_moe.h.

Loads libcco_moe.so from this package directory.  There is no fallback:
if the library is missing, importing raises, naming the build command.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcco_moe.so")

CCO_OK = 0
CCO_INFO_COPIED = 1
CCO_ERR_INVALID_ARG = -1
CCO_ERR_OUT_OF_MEMORY = -2
CCO_ERR_HIP = -3
CCO_ERR_CAPACITY = -4
CCO_ERR_BAD_EXPERT = -5
CCO_ERR_HEAP_FULL = -6
CCO_ERR_TOO_LARGE = -7
CCO_ERR_TIMEOUT = -8
CCO_ERR_DISABLED = -9
CCO_NUM_KERNEL_KINDS = 10
KERNEL_KINDS = ("plan_count", "plan_rank", "dispatch", "expert_gate_up", "expert_down",
                "combine", "combine_copy_in", "dispatch_fp8", "stage_in_sdma", "fused")


class cco_moe_shape(ctypes.Structure):
    _fields_ = [("max_tokens", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("topk", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("inter", ctypes.c_int32)]


class cco_moe_routing(ctypes.Structure):
    _fields_ = [("pos", ctypes.c_void_p), ("counts", ctypes.c_void_p),
                ("expert_off", ctypes.c_void_p), ("slot_total", ctypes.c_void_p),
                ("status", ctypes.c_void_p)]


class cco_moe_layout(ctypes.Structure):
    _fields_ = [("disp_x", ctypes.c_uint64), ("disp_x_bytes", ctypes.c_uint64),
                ("disp_meta", ctypes.c_uint64), ("disp_meta_bytes", ctypes.c_uint64),
                ("hbuf", ctypes.c_uint64), ("hbuf_bytes", ctypes.c_uint64),
                ("out_tok", ctypes.c_uint64), ("out_tok_bytes", ctypes.c_uint64),
                ("cap", ctypes.c_int64)]


# (name, restype, argtypes) for every symbol the header declares
P, I32, U64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64
PP = ctypes.POINTER(ctypes.c_void_p)
SIGNATURES = [
    ("cco_sym_heap_create", ctypes.c_int, [ctypes.c_int, I32, U64, PP]),
    ("cco_sym_heap_destroy", ctypes.c_int, [P]),
    ("cco_sym_heap_slot_ptr", P, [P, I32, U64]),
    ("cco_sym_heap_info", ctypes.c_int, [P, PP, ctypes.POINTER(U64), ctypes.POINTER(I32),
                                         ctypes.POINTER(U64)]),
    ("cco_moe_required_slot_bytes", U64, [ctypes.POINTER(cco_moe_shape), I32]),
    ("cco_moe_layout_of", ctypes.c_int, [ctypes.POINTER(cco_moe_shape), I32,
                                         ctypes.POINTER(cco_moe_layout)]),
    ("cco_moe_create", ctypes.c_int, [P, ctypes.POINTER(cco_moe_shape), PP]),
    ("cco_moe_get_layout", ctypes.c_int, [P, ctypes.POINTER(cco_moe_layout)]),
    ("cco_moe_get_routing", ctypes.c_int, [P, ctypes.POINTER(cco_moe_routing)]),
    ("cco_moe_plan", ctypes.c_int, [P, P, I32, P]),
    ("cco_moe_dispatch", ctypes.c_int, [P, P, P, I32, P]),
    ("cco_moe_dispatch_fp8", ctypes.c_int, [P, P, P, I32, P, I32, P]),
    ("cco_moe_expert", ctypes.c_int, [P, P, P, P]),
    ("cco_moe_dispatch_view", P, [P, I32]),
    ("cco_moe_combine_in_view", P, [P, I32]),
    ("cco_moe_combine", ctypes.c_int, [P, P, P, P, I32, P]),
    ("cco_moe_fused", ctypes.c_int, [P, P, P, P, P, P, P, I32, P]),
    ("cco_moe_stage_in_sdma", ctypes.c_int, [P, I32, P, I32, P]),
    ("cco_moe_status", ctypes.c_int, [P, P, P, P]),
    ("cco_moe_set_timing", ctypes.c_int, [P, ctypes.c_int]),
    ("cco_moe_timing_summary", ctypes.c_int, [P, P, P]),
    ("cco_moe_plan_noalloc", ctypes.c_int, [P, I32, I32, I32, I32, ctypes.c_int64, P, P, P,
                                             P, P, P]),
    ("cco_status_string", ctypes.c_char_p, [ctypes.c_int]),
]


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(
            "libcco_moe.so not found at %s; build it with "
            "`python combine_symmetric_memory_amd/build.py` (hipcc, gfx950)" % path)
    lib = ctypes.CDLL(path)
    for name, res, args in SIGNATURES:
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = load()


class CcoError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__("%s failed: %s (%d)" % (where, status_string(code), code))


def status_string(code: int) -> str:
    return lib.cco_status_string(code).decode()


def check(code: int, where: str, allow=(CCO_OK,)) -> int:
    if code not in allow:
        raise CcoError(code, where)
    return code
