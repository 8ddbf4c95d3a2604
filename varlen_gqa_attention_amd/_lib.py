"""ctypes loader for libvattn.so (the C ABI declared in include/vattn.h).

Argument marshalling only: every step of the computation runs in the HIP
library. If the library is missing this module raises at import time; there
is no fallback.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libvattn.so")

VATTN_OK = 0
VATTN_ERR_INVALID_ARG = -1
VATTN_ERR_UNSUPPORTED = -2
VATTN_ERR_HIP = -3
VATTN_ERR_OOM = -4
VATTN_ERR_TOO_LARGE = -5

DECODE_AUTO, DECODE_WAVE, DECODE_MFMA = 0, 1, 2
ERRBIT_Q_LEN, ERRBIT_KV_LEN, ERRBIT_ROWS, ERRBIT_INDEX = 0x1, 0x2, 0x4, 0x8

# every symbol include/vattn.h declares
EXPORTS = (
    "vattn_status_string", "vattn_abi_version", "vattn_plan", "vattn_plan_ex",
    "vattn_plan_describe", "vattn_plan_query", "vattn_execute", "vattn_execute_gathered",
    "vattn_execute_strided", "vattn_backward",
    "vattn_execute_exact_grid", "vattn_padding_mask", "vattn_cross_padding_mask",
    "vattn_plan_error_word",
    "vattn_plan_read_error", "vattn_plan_clear_error", "vattn_plan_set_kernel_events",
    "vattn_plan_destroy", "vattn_execute_noalloc",
)


class PlanOpts(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in (
        "target_blocks_per_cu", "nsplit_cap", "force_nsplit", "force_decode_path",
        "n_cu_override", "fuse_combine", "decode_waves", "prefill_grid", "backward",
        "min_chunk_tiles")]


_INFO_INT_FIELDS = (
    "B_max", "s_max_q", "s_max_kv", "Hq", "Hkv", "D", "causal", "is_decode", "decode_path",
    "n_cu", "block_n", "n_tiles", "nsplit", "chunk_keys", "direct", "fused_combine",
    "head_blocks", "n_units", "grid", "combine_grid", "q_tokens_per_tile", "n_qtiles",
    "threads", "prefill_persistent", "backward", "bwd_q_tokens_per_tile", "bwd_grid_dq",
    "bwd_grid_dkdv")


class PlanInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in _INFO_INT_FIELDS] + [("scratch_bytes", ctypes.c_longlong)]

    def as_dict(self):
        d = {n: getattr(self, n) for n in _INFO_INT_FIELDS}
        d["scratch_bytes"] = self.scratch_bytes
        return d


class VattnError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


_lib = None


def load():
    """Load the library (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python -m varlen_gqa_attention_amd.build)")
    L = ctypes.CDLL(LIB_PATH)
    c_int, c_i64, vp = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p
    i32p = ctypes.POINTER(ctypes.c_int32)
    L.vattn_status_string.restype = ctypes.c_char_p
    L.vattn_status_string.argtypes = [c_int]
    L.vattn_abi_version.restype = c_int
    L.vattn_abi_version.argtypes = []
    L.vattn_plan.restype = c_int
    L.vattn_plan.argtypes = [ctypes.POINTER(vp)] + [c_int] * 7
    L.vattn_plan_ex.restype = c_int
    L.vattn_plan_ex.argtypes = [ctypes.POINTER(vp)] + [c_int] * 7 + [ctypes.POINTER(PlanOpts)]
    L.vattn_plan_describe.restype = c_int
    L.vattn_plan_describe.argtypes = [c_int] * 7 + [ctypes.POINTER(PlanOpts), ctypes.POINTER(PlanInfo)]
    L.vattn_plan_query.restype = c_int
    L.vattn_plan_query.argtypes = [vp, ctypes.POINTER(PlanInfo)]
    L.vattn_execute.restype = c_int
    L.vattn_execute.argtypes = [vp, c_int, vp, vp, vp, vp, vp, vp, vp, c_i64, c_i64, vp]
    L.vattn_execute_gathered.restype = c_int
    L.vattn_execute_gathered.argtypes = [vp, c_int, vp, vp, vp, vp, vp, vp, vp, vp, c_i64, c_i64,
                                         c_i64, vp]
    L.vattn_execute_strided.restype = c_int
    L.vattn_execute_strided.argtypes = [vp, c_int, vp, c_i64, vp, c_i64, vp, c_i64, vp, vp, vp,
                                        c_i64, vp, c_i64, c_i64, vp]
    L.vattn_backward.restype = c_int
    L.vattn_backward.argtypes = [vp, c_int] + [vp, c_i64] * 5 + [vp, vp, vp] + [vp, c_i64] * 3 + \
        [c_i64, c_i64, vp]
    L.vattn_execute_exact_grid.restype = c_int
    L.vattn_execute_exact_grid.argtypes = [vp, c_int, vp, vp, vp, vp, vp, vp, vp, c_i64, c_i64,
                                           vp, c_int, vp]
    L.vattn_padding_mask.restype = c_int
    L.vattn_padding_mask.argtypes = [vp, c_int, c_int, vp, vp]
    L.vattn_cross_padding_mask.restype = c_int
    L.vattn_cross_padding_mask.argtypes = [vp, vp, c_int, c_int, c_int, vp, vp, vp]
    L.vattn_plan_error_word.restype = vp
    L.vattn_plan_error_word.argtypes = [vp]
    L.vattn_plan_read_error.restype = c_int
    L.vattn_plan_read_error.argtypes = [vp, i32p]
    L.vattn_plan_clear_error.restype = c_int
    L.vattn_plan_clear_error.argtypes = [vp, vp]
    L.vattn_plan_set_kernel_events.restype = c_int
    L.vattn_plan_set_kernel_events.argtypes = [vp, vp, vp]
    L.vattn_plan_destroy.restype = None
    L.vattn_plan_destroy.argtypes = [vp]
    L.vattn_execute_noalloc.restype = c_int
    L.vattn_execute_noalloc.argtypes = [c_int] * 8 + [vp] * 7 + [c_i64, c_i64, vp, vp]
    _lib = L
    return L


def status_string(status):
    try:
        return load().vattn_status_string(int(status)).decode()
    except ImportError:
        return "status"


def check(status, what):
    if status != VATTN_OK:
        raise VattnError(status, what)
