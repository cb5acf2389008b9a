"""ctypes declarations of the C ABI in include/hyq.h (argument marshalling only)."""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhyq.so")

HYQ_OK = 0
STATUS = {0: "HYQ_OK", 1: "HYQ_ERR_INVALID", 2: "HYQ_ERR_UNSUPPORTED", 3: "HYQ_ERR_CAPACITY",
          4: "HYQ_ERR_WORKSPACE", 5: "HYQ_ERR_HIP"}
HYQ_OP_DECODE, HYQ_OP_SELECT, HYQ_OP_PREFILL, HYQ_OP_SELECT_TAIL = 1, 2, 3, 4
HYQ_NOALLOC_SCRATCH_BYTES = 8 << 20
HYQ_NBUF = 10
BUFFERS = ["int4", "slot_pos", "a_k", "a_v", "a_pos", "s_k", "s_v", "w_k", "w_v", "proxy_q"]

# every symbol include/hyq.h declares
EXPORTS = ["hyq_status_string", "hyq_cache_buffer_bytes", "hyq_workspace_bytes", "hyq_quantize_kv",
           "hyq_append_token", "hyq_select_vlines", "hyq_decode_attn", "hyq_prefill_attn",
           "hyq_prefill_attn_mx", "hyq_select_vlines_tail", "hyq_decode_attn_ragged",
           "hyq_decode_ragged_workspace_bytes", "hyq_decode_ragged_table_bytes", "hyq_decode_ragged_plan", "hyq_decode_attn_noalloc"]


class HyqShape(C.Structure):
    _fields_ = [("batch", C.c_int32), ("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("group", C.c_int32), ("window", C.c_int32),
                ("proxy_cap", C.c_int32), ("staging_cap", C.c_int32), ("int4_cap", C.c_int32),
                ("anchor_cap", C.c_int32), ("bits", C.c_int32), ("bits_v", C.c_int32)]


class HyqCache(C.Structure):
    _fields_ = [("shape", HyqShape)] + [(n, C.c_void_p) for n in BUFFERS] + [
        ("len", C.c_int32), ("n_int4", C.c_int32), ("n_anchor", C.c_int32), ("n_staged", C.c_int32),
        ("n_proxy", C.c_int32), ("proxy_head", C.c_int32)]


_lib = None


class HyqError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}")
        self.status = status


def load() -> C.CDLL:
    """Load the built library; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: run `python -m hybrid_precision_kv_amd.build` "
                          "(the HIP library is required; there is no CPU fallback)")
    lib = C.CDLL(LIB_PATH)
    vp, i32, sz = C.c_void_p, C.c_int32, C.c_size_t
    lib.hyq_status_string.restype = C.c_char_p
    lib.hyq_status_string.argtypes = [C.c_int]
    lib.hyq_cache_buffer_bytes.restype = C.c_int
    lib.hyq_cache_buffer_bytes.argtypes = [C.POINTER(HyqShape), C.POINTER(C.c_size_t * HYQ_NBUF)]
    lib.hyq_workspace_bytes.restype = sz
    lib.hyq_workspace_bytes.argtypes = [C.POINTER(HyqShape), C.c_int, i32, i32]
    lib.hyq_quantize_kv.restype = C.c_int
    lib.hyq_quantize_kv.argtypes = [C.POINTER(HyqCache), vp, vp, i32, vp, i32, vp, i32, vp]
    lib.hyq_append_token.restype = C.c_int
    lib.hyq_append_token.argtypes = [C.POINTER(HyqCache), vp, vp, vp, vp]
    lib.hyq_select_vlines.restype = C.c_int
    lib.hyq_select_vlines.argtypes = [C.POINTER(HyqShape), C.POINTER(HyqCache), vp, i32, vp, i32, i32, i32,
                                      vp, vp, vp, sz, vp]
    lib.hyq_decode_attn.restype = C.c_int
    lib.hyq_decode_attn.argtypes = [C.POINTER(HyqCache), vp, vp, i32, vp, sz, vp]
    lib.hyq_decode_attn_noalloc.restype = C.c_int
    lib.hyq_decode_attn_noalloc.argtypes = [C.POINTER(HyqCache), vp, vp, i32, vp]
    lib.hyq_prefill_attn.restype = C.c_int
    lib.hyq_prefill_attn.argtypes = [C.POINTER(HyqShape), vp, vp, vp, i32, vp, i32, vp, vp, sz, vp]
    lib.hyq_select_vlines_tail.restype = C.c_int
    lib.hyq_select_vlines_tail.argtypes = [C.POINTER(HyqShape), vp, i32, vp, i32, i32, vp, vp, vp, sz, vp]
    lib.hyq_decode_attn_ragged.restype = C.c_int
    lib.hyq_decode_attn_ragged.argtypes = [C.POINTER(C.POINTER(HyqCache)), i32, vp, vp, i32, vp, sz, vp, sz, vp]
    lib.hyq_decode_ragged_workspace_bytes.restype = sz
    lib.hyq_decode_ragged_workspace_bytes.argtypes = [C.POINTER(HyqShape), i32, i32]
    lib.hyq_decode_ragged_table_bytes.restype = sz
    lib.hyq_decode_ragged_table_bytes.argtypes = [C.POINTER(HyqShape), i32, i32]
    lib.hyq_decode_ragged_plan.restype = C.c_int
    lib.hyq_decode_ragged_plan.argtypes = [C.POINTER(C.POINTER(HyqCache)), i32, i32, vp, sz, C.POINTER(i32)]
    lib.hyq_prefill_attn_mx.restype = C.c_int
    lib.hyq_prefill_attn_mx.argtypes = [C.POINTER(HyqShape), vp, vp, vp, i32, vp, i32, vp, vp, sz, vp]
    _lib = lib
    return lib


def check(fn: str, status: int) -> None:
    if status != HYQ_OK:
        raise HyqError(fn, status)
