"""ctypes loader for ``libtopk_select.so`` (the C ABI in ``include/topk_select.h``).

Argument marshalling only: every step of the selection runs in the HIP
kernels of the library.  There is no fallback: if the library is missing or
fails to load, every entry point raises.
"""

from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libtopk_select.so")

SUCCESS = 0
ERROR_INVALID_VALUE = 1
ERROR_OUT_OF_MEMORY = 2
ERROR_LAUNCH = 3
ERROR_NO_DEVICE = 4
ERROR_DEVICE_FLAG = 5
ERROR_CAPTURE = 6
ERROR_SCRATCH_LIMIT = 7

# Names declared in include/topk_select.h.
EXPORTS = (
    "topk_select",
    "topk_select_ex",
    "topk_select_no_alloc",
    "topk_select_sorted",
    "topk_select_sorted_ex",
    "topk_indexer_logits",
    "topk_indexer_select",
    "topk_indexer_select_fused",
    "topk_sparse_attention",
    "topk_select_plan",
    "topk_select_num_variants",
    "topk_select_variant_info",
    "topk_select_device_status",
    "topk_select_release_workspace",
    "topk_select_error_string",
    "topk_select_version",
    "topk_stream_read",
)


class PlanT(ctypes.Structure):
    _fields_ = [
        ("variant", ctypes.c_int32),
        ("wgs_per_row", ctypes.c_int32),
        ("block", ctypes.c_int32),
        ("items", ctypes.c_int32),
        ("resident", ctypes.c_int32),
        ("first_bits", ctypes.c_int32),
    ]


class TopkSelectError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__("%s: status %d (%s)" % (what or "topk_select", status, error_string(status)))


_lock = threading.Lock()
_lib = None


def load() -> ctypes.CDLL:
    """Load the built library (raises when it is absent)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                "libtopk_select.so is not built (expected at %s); run "
                "`python -m sparse_attention_topk_fp32_amd.build`" % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        P, I = ctypes.c_void_p, ctypes.c_int32
        lib.topk_select.argtypes = [P, I, I, P, I, P, P]
        lib.topk_select.restype = ctypes.c_int
        lib.topk_select_ex.argtypes = [P, I, I, P, I, P, P, ctypes.POINTER(PlanT)]
        lib.topk_select_ex.restype = ctypes.c_int
        lib.topk_select_no_alloc.argtypes = [P, I, I, P, I, P, P]
        lib.topk_select_no_alloc.restype = ctypes.c_int
        lib.topk_select_sorted.argtypes = [P, I, I, P, I, P, P, P]
        lib.topk_select_sorted.restype = ctypes.c_int
        lib.topk_select_sorted_ex.argtypes = [P, I, I, P, I, P, P, P, ctypes.POINTER(PlanT)]
        lib.topk_select_sorted_ex.restype = ctypes.c_int
        I64 = ctypes.c_int64
        lib.topk_indexer_logits.argtypes = [P, P, P, I, I, I, I, I64, P, P, P]
        lib.topk_indexer_logits.restype = ctypes.c_int
        lib.topk_indexer_select.argtypes = [P, P, P, I, I, I, I, I64, P, I, P, P, P]
        lib.topk_indexer_select.restype = ctypes.c_int
        lib.topk_indexer_select_fused.argtypes = [P, P, P, I, I, I, I, I64, P, I, P, P, P]
        lib.topk_indexer_select_fused.restype = ctypes.c_int
        lib.topk_sparse_attention.argtypes = [P, P, P, P, I, I, I, I, I64, I, ctypes.c_float, P, P]
        lib.topk_sparse_attention.restype = ctypes.c_int
        lib.topk_select_plan.argtypes = [I, I, I, ctypes.POINTER(PlanT)]
        lib.topk_select_plan.restype = ctypes.c_int
        lib.topk_select_num_variants.argtypes = []
        lib.topk_select_num_variants.restype = ctypes.c_int
        lib.topk_select_variant_info.argtypes = [I, ctypes.POINTER(PlanT)]
        lib.topk_select_variant_info.restype = ctypes.c_int
        lib.topk_select_device_status.argtypes = [P, ctypes.POINTER(ctypes.c_int32)]
        lib.topk_select_device_status.restype = ctypes.c_int
        lib.topk_select_release_workspace.argtypes = []
        lib.topk_select_release_workspace.restype = ctypes.c_int
        lib.topk_select_error_string.argtypes = [ctypes.c_int]
        lib.topk_select_error_string.restype = ctypes.c_char_p
        lib.topk_select_version.argtypes = []
        lib.topk_select_version.restype = ctypes.c_int
        lib.topk_stream_read.argtypes = [P, ctypes.c_size_t, P, P]
        lib.topk_stream_read.restype = ctypes.c_int
        _lib = lib
        return lib


def error_string(status: int) -> str:
    try:
        return load().topk_select_error_string(int(status)).decode()
    except Exception:  # the library itself failed to load
        return "unknown"
