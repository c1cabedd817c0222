"""ctypes view of librpe_attn.so (declared in include/rpe_attn.h).

Argument marshalling only.  The library is loaded on first use; if it is not
built the call raises: there is no other implementation to fall back to.
"""

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "librpe_attn.so")

RPE_OK = 0
RPE_BF16, RPE_FP32 = 0, 1
RPE_MODE_NONE, RPE_MODE_BIAS, RPE_MODE_CONTEXTUAL = 0, 1, 2
RPE_TERM_K, RPE_TERM_Q, RPE_TERM_V = 1, 2, 4
RPE_MAP_SWIN, RPE_MAP_PIECEWISE = 0, 1
RPE_MAP_EUCLIDEAN, RPE_MAP_EUCLIDEAN_ROUNDED, RPE_MAP_QUANTIZED, RPE_MAP_QUANTIZED_SQUARED = 2, 3, 4, 5
RPE_ROUND_CAPPED, RPE_ROUND_TRUNC = 0, 1
RPE_TABLE_BIAS, RPE_TABLE_VECTOR = 0, 1
RPE_METHOD_PRODUCT, RPE_METHOD_CROSS = 0, 1

STATUS_NAMES = {
    0: "RPE_OK", -1: "RPE_E_NULL", -2: "RPE_E_SHAPE", -3: "RPE_E_DTYPE", -4: "RPE_E_MODE",
    -5: "RPE_E_BIAS_ON_VALUES", -6: "RPE_E_BUCKETS", -7: "RPE_E_PARAMS", -8: "RPE_E_UNSUPPORTED",
    -9: "RPE_E_HIP", -10: "RPE_E_ALIGN",
}

# Every symbol include/rpe_attn.h declares.
EXPORTS = ("rpe_attn_validate", "rpe_attn_num_buckets", "rpe_attn_unit_size", "rpe_attn_axis_index",
           "rpe_attn_bucket_map", "rpe_attn_cross_to_product", "rpe_attn_undirected_to_product", "rpe_attn_fwd",
           "rpe_attn_fwd_plan",
           "rpe_attn_bwd_workspace_size", "rpe_attn_bwd", "rpe_attn_bwd_noalloc", "rpe_status_str",
           "rpe_attn_version")
BWD_NOALLOC_MAX_BYTES = 64 << 20


class Desc(ctypes.Structure):
    """Mirror of ``rpe_attn_desc``."""

    _fields_ = [
        ("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("grid_h", ctypes.c_int32), ("grid_w", ctypes.c_int32), ("window", ctypes.c_int32),
        ("prefix_tokens", ctypes.c_int32), ("dtype", ctypes.c_int32), ("mode", ctypes.c_int32),
        ("terms", ctypes.c_uint32), ("map", ctypes.c_int32), ("rounding", ctypes.c_int32),
        ("alpha", ctypes.c_double), ("beta", ctypes.c_double), ("gamma", ctypes.c_double),
        ("scale", ctypes.c_float), ("tables_per_head", ctypes.c_int32), ("method", ctypes.c_int32),
        ("table_head_stride", ctypes.c_int64),
        ("stride_b", ctypes.c_int64), ("stride_h", ctypes.c_int64), ("stride_n", ctypes.c_int64),
        ("o_stride_b", ctypes.c_int64), ("o_stride_h", ctypes.c_int64), ("o_stride_n", ctypes.c_int64),
    ]


class RpeError(RuntimeError):
    def __init__(self, fn, status, text):
        super().__init__(f"{fn} failed: {STATUS_NAMES.get(status, status)} ({text})")
        self.status = status


class PlanInfo(ctypes.Structure):
    """Mirror of ``rpe_attn_plan_info``."""

    _fields_ = [
        ("row_slots", ctypes.c_int32),
        ("key_blocks", ctypes.c_int32),
        ("waves_per_group", ctypes.c_int32),
        ("query_chunks", ctypes.c_int32),
        ("units_per_group", ctypes.c_int32),
        ("ring_stages", ctypes.c_int32),
        ("lds_bytes", ctypes.c_int32),
        ("waves_per_simd", ctypes.c_int32),
        ("value_term", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("workgroups", ctypes.c_int64),
    ]


_lib = None
_lock = threading.Lock()


def load():
    """Load the library (once) and declare the signatures."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m vision_transformer_attention_amd.build` "
                "(or __graft_entry__.build()) first")
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        vp = ctypes.c_void_p
        i32 = ctypes.c_int32
        lib.rpe_attn_validate.argtypes = [P(Desc)]
        lib.rpe_attn_validate.restype = i32
        lib.rpe_attn_num_buckets.argtypes = [P(Desc), P(i32), P(i32), P(i32)]
        lib.rpe_attn_num_buckets.restype = i32
        lib.rpe_attn_unit_size.argtypes = [P(Desc), P(i32), P(i32), P(i32)]
        lib.rpe_attn_unit_size.restype = i32
        lib.rpe_attn_axis_index.argtypes = [P(Desc), i32, vp, vp]
        lib.rpe_attn_axis_index.restype = i32
        lib.rpe_attn_bucket_map.argtypes = [P(Desc), vp, vp]
        lib.rpe_attn_bucket_map.restype = i32
        lib.rpe_attn_cross_to_product.argtypes = [P(Desc), i32, vp, vp, vp]
        lib.rpe_attn_cross_to_product.restype = i32
        lib.rpe_attn_undirected_to_product.argtypes = [P(Desc), i32, vp, vp, vp]
        lib.rpe_attn_undirected_to_product.restype = i32
        lib.rpe_attn_fwd.argtypes = [P(Desc), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.rpe_attn_fwd_plan.argtypes = [P(Desc), P(PlanInfo)]
        lib.rpe_attn_fwd_plan.restype = i32
        lib.rpe_attn_bwd_workspace_size.argtypes = [P(Desc), P(ctypes.c_uint64)]
        lib.rpe_attn_bwd_workspace_size.restype = i32
        lib.rpe_attn_bwd.argtypes = [P(Desc)] + [vp] * 17 + [ctypes.c_uint64, vp]
        lib.rpe_attn_bwd.restype = i32
        lib.rpe_attn_bwd_noalloc.argtypes = [P(Desc)] + [vp] * 16 + [vp]
        lib.rpe_attn_bwd_noalloc.restype = i32
        lib.rpe_attn_fwd.restype = i32
        lib.rpe_status_str.argtypes = [i32]
        lib.rpe_status_str.restype = ctypes.c_char_p
        lib.rpe_attn_version.argtypes = []
        lib.rpe_attn_version.restype = ctypes.c_char_p
        _lib = lib
        return lib


def check(fn, status):
    if status != RPE_OK:
        raise RpeError(fn, status, load().rpe_status_str(status).decode())
    return status
