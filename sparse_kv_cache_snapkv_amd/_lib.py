"""ctypes loader for librkv.so. There is no fallback: a missing library is an error."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librkv.so")

_c_int, _c_float, _c_size, _vp = ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p
_szp = ctypes.POINTER(ctypes.c_size_t)

# name -> (restype, argtypes); mirrors include/rkv.h
SIGNATURES = {
    "rkv_version": (_c_int, []),
    "rkv_status_string": (ctypes.c_char_p, [_c_int]),
    "rkv_plan_budget": (_c_int, [_c_int] * 4 + [ctypes.POINTER(_c_int)] * 6),
    "rkv_snapkvpp_workspace_bytes": (_c_int, [_c_int] * 8 + [_szp]),
    "rkv_snapkvpp_evict": (_c_int, [_vp, _vp, _vp] + [_c_int] * 9 + [_c_float, _c_int]
                           + [_vp, _vp, _vp, _vp, _vp, _c_size, _vp]),
    "rkv_build_page_summaries": (_c_int, [_vp] + [_c_int] * 6 + [_vp, _vp, _vp]),
    "rkv_hybrid_approx_scores": (_c_int, [_vp, _vp, _vp] + [_c_int] * 7 + [_vp, _vp, _vp]),
    "rkv_topk_workspace_bytes": (_c_int, [_c_int] * 3 + [_szp]),
    "rkv_topk_select": (_c_int, [_vp, _c_int, _c_int, _c_int, _vp, _vp, _c_size, _vp]),
    "rkv_sparse_attend_workspace_bytes": (_c_int, [_c_int] * 7 + [_szp]),
    "rkv_sparse_attend_decode": (_c_int, [_vp, _vp, _vp, _vp] + [_c_int] * 7 + [_c_float, _c_int]
                                 + [_vp, _vp, _c_size, _vp]),
    "rkv_hybrid_decode_workspace_bytes": (_c_int, [_c_int] * 8 + [_szp]),
    "rkv_hybrid_decode_workspace_init": (_c_int, [_vp, _c_size, _vp]),
    "rkv_hybrid_decode_status": (_c_int, [_vp, _c_size, _c_int, ctypes.POINTER(ctypes.c_uint32),
                                          _vp]),
    "rkv_hybrid_decode_step": (_c_int, [_vp] * 5 + [_c_int] * 8 + [_c_float, _c_int]
                               + [_vp, _vp, _vp, _vp, _vp, _c_size, _vp]),
    "rkv_hybrid_decode_step_noalloc": (_c_int, [_vp] * 5 + [_c_int] * 8 + [_c_float, _c_int]
                                       + [_vp, _vp, _vp, _vp, _vp, _vp]),
    "rkv_build_page_summaries_cap": (_c_int, [_vp] + [_c_int] * 7 + [_vp, _vp, _vp]),
    "rkv_kv_append": (_c_int, [_vp, _vp] + [_c_int] * 7 + [_vp, _vp, _vp, _vp, _vp]),
    "rkv_hybrid_decode_step_cap": (_c_int, [_vp] * 5 + [_c_int] * 9 + [_c_float, _c_int]
                                   + [_vp, _vp, _vp, _vp, _vp, _c_size, _vp]),
    "rkv_build_page_summaries_indexed": (_c_int, [_vp, _vp] + [_c_int] * 7 + [_vp, _vp, _vp]),
    "rkv_hybrid_decode_step_indexed": (_c_int, [_vp] * 6 + [_c_int] * 9 + [_c_float, _c_int]
                                       + [_vp, _vp, _vp, _vp, _vp, _c_size, _vp]),
}

_lib = None


def load() -> ctypes.CDLL:
    """The loaded library with argument types set; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m sparse_kv_cache_snapkv_amd.build` "
            "(the RocketKV path has no CPU fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib
