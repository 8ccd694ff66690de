"""ctypes view of libcsa2.so (the C ABI declared in include/csa2.h).

The library is loaded on first use. There is no fallback: if the shared object is missing or
fails to load, every call raises.
"""
from __future__ import annotations

import ctypes as C
import os
import threading

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcsa2.so")

STATUS = {
    0: "CSA2_OK",
    1: "CSA2_E_ARG",
    2: "CSA2_E_SHAPE",
    3: "CSA2_E_STATE",
    4: "CSA2_E_WORKSPACE",
    5: "CSA2_E_UNSUPPORTED",
    6: "CSA2_E_HIP",
}

EXPORTS = [
    "csa2_status_string",
    "csa2_quantize_kv_fp4",
    "csa2_dequant_kv_fp4",
    "csa2_compress_kv",
    "csa2_index_scores",
    "csa2_prefill_visibility",
    "csa2_topk_workspace_size",
    "csa2_topk",
    "csa2_hier_pool_workspace_size",
    "csa2_hier_pool",
    "csa2_sparse_attn_workspace_size",
    "csa2_sparse_attn",
    "csa2_sparse_attn_swa_workspace_size",
    "csa2_sparse_attn_swa",
    "csa2_sparse_attn_swa_prefill_workspace_size",
    "csa2_sparse_attn_swa_prefill",
    "csa2_index_scores_mxfp4",
    "csa2_layer_workspace_size",
    "csa2_layer_step",
    "csa2_layer_step_noalloc",
]


class Csa2Error(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed: {STATUS.get(code, code)} ({msg})")
        self.code = code


class SharedKV(C.Structure):
    _fields_ = [("rows", C.c_void_p), ("k_idx", C.c_void_p), ("n_vis", C.c_void_p),
                ("B", C.c_int32), ("n_max", C.c_int32), ("D", C.c_int32), ("Hk", C.c_int32),
                ("Di", C.c_int32), ("valid", C.c_int32), ("k_mx", C.c_void_p)]


class SharedIdx(C.Structure):
    _fields_ = [("topk", C.c_void_p), ("K", C.c_int32), ("pool", C.c_void_p), ("P", C.c_int32),
                ("topk_valid", C.c_int32), ("pool_valid", C.c_int32)]


class LayerArgs(C.Structure):
    _fields_ = [("q", C.c_void_p), ("q_idx", C.c_void_p), ("T", C.c_int32), ("H", C.c_int32),
                ("Hi", C.c_int32), ("sm_scale", C.c_float), ("use_pool", C.c_int32),
                ("pool_blocks", C.c_int32), ("block", C.c_int32), ("out", C.c_void_p),
                ("lse", C.c_void_p), ("ws", C.c_void_p), ("ws_bytes", C.c_size_t),
                ("swa_codes", C.c_void_p), ("swa_exp", C.c_void_p), ("swa_n", C.c_void_p), ("swa_W", C.c_int32),
                ("q_idx_mx", C.c_void_p), ("new_kv", C.c_void_p), ("new_z", C.c_void_p), ("new_tokens", C.c_int32),
                ("ratio", C.c_int32), ("new_entry0", C.c_void_p), ("w_ik", C.c_void_p)]


_lib = None
_lock = threading.Lock()


def _declare(lib):
    vp, i32, i64, sz, f32 = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t, C.c_float
    sig = {
        "csa2_status_string": (C.c_char_p, [i32]),
        "csa2_quantize_kv_fp4": (i32, [vp, i32, i64, i32, vp, vp]),
        "csa2_dequant_kv_fp4": (i32, [vp, i64, i32, vp, vp]),
        "csa2_compress_kv": (i32, [vp, vp, i32, i32, i32, i32, vp, i32, vp, vp, i32, i32, vp, vp, vp]),
        "csa2_index_scores": (i32, [vp, vp, i32, i32, i32, i32, i32, i32, vp, vp, i32, vp, vp, i32, vp]),
        "csa2_prefill_visibility": (i32, [vp, i32, i32, i32, i32, vp, vp]),
        "csa2_topk_workspace_size": (sz, [i64, i32, i32]),
        "csa2_topk": (i32, [vp, i64, i32, vp, vp, i32, vp, vp, sz, vp]),
        "csa2_hier_pool_workspace_size": (sz, [i64, i32, i32]),
        "csa2_hier_pool": (i32, [vp, i64, i32, vp, i32, i32, vp, vp, sz, vp]),
        "csa2_sparse_attn_workspace_size": (sz, [i32, i32, i32, i32, i32]),
        "csa2_sparse_attn": (i32, [vp, vp, i32, vp, i32, i32, i32, i32, i32, f32, vp, vp, vp, sz, vp]),
        "csa2_sparse_attn_swa_workspace_size": (sz, [i32, i32, i32, i32]),
        "csa2_sparse_attn_swa": (i32, [vp, vp, i32, vp, i32, i32, i32, i32, vp, vp, vp, i32, f32, vp, vp, vp, sz, vp]),
        "csa2_sparse_attn_swa_prefill_workspace_size": (sz, [i32, i32, i32, i32, i32]),
        "csa2_sparse_attn_swa_prefill": (i32, [vp, vp, i32, vp, i32, i32, i32, i32, i32, vp, vp, vp, i32, f32, vp, vp,
                                               vp, sz, vp]),
        "csa2_index_scores_mxfp4": (i32, [vp, vp, i32, i32, i32, i32, i32, i32, vp, vp, i32, vp, vp, i32, vp]),
        "csa2_layer_workspace_size": (i32, [i32, C.POINTER(LayerArgs), C.POINTER(SharedKV),
                                            C.POINTER(SharedIdx), C.POINTER(sz)]),
        "csa2_layer_step": (i32, [i32, C.POINTER(LayerArgs), C.POINTER(SharedKV), C.POINTER(SharedIdx), vp]),
        "csa2_layer_step_noalloc": (i32, [i32, C.POINTER(LayerArgs), C.POINTER(SharedKV), C.POINTER(SharedIdx), vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args


def lib():
    """The loaded library; raises if libcsa2.so has not been built."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise RuntimeError(
                        f"{LIB_PATH} is missing: build it with `python -m fp4_kv_cache_e2m1_amd.build_lib` "
                        "(there is no non-HIP fallback)")
                l = C.CDLL(LIB_PATH)
                _declare(l)
                _lib = l
    return _lib


def check(fn_name: str, code: int):
    if code != 0:
        msg = lib().csa2_status_string(code).decode()
        raise Csa2Error(fn_name, code, msg)
