"""ctypes loader for libdbs.so and the argument types of every C-ABI entry point.

The library is the one build.py writes into this package directory (or the
build that DBS_LIB_PATH names); a missing library raises RuntimeError, and
there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes as C
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
# DBS_LIB_PATH selects another build of the same library (the host-sanitizer
# build that the CPU tests load); by default the one built in this directory.
LIB_PATH = os.environ.get("DBS_LIB_PATH") or os.path.join(_HERE, "libdbs.so")

DBS_OK = 0
STATUS_NAMES = {0: "DBS_OK", -1: "DBS_ERR_INVALID_ARG", -2: "DBS_ERR_UNSUPPORTED",
                -3: "DBS_ERR_ALIGNMENT", -4: "DBS_ERR_LAUNCH", -5: "DBS_ERR_HIP"}
DBS_BF16, DBS_FP32 = 0, 1
DBS_ROWS, DBS_TILES_T = 0, 1

_i32p = C.POINTER(C.c_int32)
_vp = C.c_void_p
_i = C.c_int
_i64 = C.c_int64
_f = C.c_float

# name -> (restype, argtypes)
SIGNATURES = {
    "dbs_abi_version": (C.c_int, []),
    "dbs_last_error": (C.c_char_p, []),
    "dbs_perm_gilbert3d": (_i, [_i, _i, _i, _i, _vp]),
    "dbs_perm_cuboid": (_i, [_i, _i, _i, _i, _i, _i, _i, _vp]),
    "dbs_perm_invert": (_i, [_vp, _i, _vp]),
    "dbs_reorder": (_i, [_vp, _i, _i64, _i64, _i64, _vp, _i, _i, _vp, _i, _i, _i, _i, _i, _i, _i, _vp]),
    "dbs_reorder_kv": (_i, [_vp, _vp, _i, _i64, _i64, _i64, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp]),
    "dbs_inverse_reorder": (_i, [_vp, _i, _vp, _i, _i64, _i64, _i64, _vp, _i, _i, _i, _i, _i, _i, _vp]),
    "dbs_estimate_workspace_bytes": (C.c_size_t, [_i, _i, _i, _i, _i, _i]),
    "dbs_estimate_blocks": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _f, _vp, _vp, C.c_size_t, _vp]),
    "dbs_estimate_blocks_tok": (_i, [_vp, _i, _i64, _i64, _i64, _vp, _i, _vp, _i, _i, _i, _i, _i, _i, _i, _f,
                                     _vp, _vp, C.c_size_t, _vp]),
    "dbs_build_mask": (_i, [_vp, _i, _i, _i, _f, _vp, _vp, _vp, _vp, _vp]),
    "dbs_build_mask_rule": (_i, [_vp, _i, _i, _i, _i, C.c_double, _vp, _vp, _vp, _vp, _vp]),
    "dbs_prune_anchors": (_i, [_i, _i, _i, _i, _i, _i, _i, _vp, _vp]),
    "dbs_query_prune": (_i, [_vp, _i, _i64, _i64, _i64, _vp, _i, _vp, _i, _i, _i, _i, _i, _i, C.c_double, _vp, _vp,
                             _vp, _vp]),
    "dbs_sparse_attn_fwd_pruned_tok": (_i, [_vp, _i, _i64, _i64, _i64, _vp, _i, _vp, _vp, _i, _i, _i, _i, _i, _i,
                                            _f, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i64, _i64, _i64, _vp,
                                            _vp]),
    "dbs_pooled_workspace_bytes": (C.c_size_t, [_i, _i, _i, _i, _i]),
    "dbs_estimate_pooled_tok": (_i, [_vp, _i, _i64, _i64, _i64, _vp, _i, _vp, _i, _i, _i, _i, _i, _i, _i, _vp, _vp,
                                     C.c_size_t, _vp]),
    "dbs_sics_tok": (_i, [_vp, _i, _i64, _i64, _i64, _vp, _i, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp]),
    "dbs_sics_choose": (_i, [_vp, _vp, _i, _i64, _i64, _i64, _vp, _i, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp,
                             _vp]),
    "dbs_normal_quantile": (C.c_double, [C.c_double]),
    "dbs_reorder_kv_pool": (_i, [_vp, _vp, _i, _i64, _i64, _i64, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i,
                                 _vp, _vp, _vp]),
    "dbs_estimate_mask": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _f, _i, C.c_double, _vp, _vp, _vp, _vp,
                               _vp, _vp, C.c_size_t, _vp]),
    "dbs_estimate_mask_tok": (_i, [_vp, _i, _i64, _i64, _i64, _vp, _i, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _i,
                                   C.c_double, _vp, _vp, _vp, _vp, _vp, _vp, C.c_size_t, _vp]),
    "dbs_estimate_mask_tok_noalloc": (_i, [_vp, _i, _i64, _i64, _i64, _vp, _i, _vp, _i, _i, _i, _i, _i, _i, _i, _f,
                                           _i, C.c_double, _vp, _vp, _vp, _vp, _vp, _vp]),
    "dbs_estimate_kvtok_workspace_bytes": (C.c_size_t, [_i, _i, _i, _i, _i, _i]),
    "dbs_estimate_mask_kvtok": (_i, [_vp, _i, _i64, _i64, _i64, _vp, _i, _i64, _i64, _i64, _vp, _i, _i, _i, _i, _i,
                                     _i, _i, _i, _f, _i, C.c_double, _vp, _vp, _vp, _vp, _vp, _vp, C.c_size_t, _vp]),
    "dbs_meanpool_kv": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp]),
    "dbs_sparse_attn_fwd": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _vp, _vp, _vp, _vp, _vp,
                                 _i, _i, _vp, _vp, _vp]),
    "dbs_sparse_attn_fwd_tok": (_i, [_vp, _i, _i64, _i64, _i64, _vp, _i, _vp, _vp, _i, _i, _i, _i, _i, _i, _f,
                                     _vp, _vp, _vp, _vp, _vp, _i, _i, _vp, _i, _i64, _i64, _i64, _vp, _vp]),
    "dbs_transpose_lists": (_i, [_vp, _vp, _i, _i, _i, _vp, _vp, _vp]),
    "dbs_attn_bwd_workspace_bytes": (C.c_size_t, [_i, _i, _i, _i]),
    "dbs_sparse_attn_bwd": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _vp, _vp, _vp, _vp,
                                 _vp, _vp, _vp, _vp, C.c_size_t, _vp]),
}

_lock = threading.Lock()
_lib = None


class DbsError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with {STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


def lib() -> C.CDLL:
    """The loaded library; raises if libdbs.so was not built."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with `python -m dynamic_block_sparse_gilbert_amd.build`")
            h = C.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(h, name)
                fn.restype = res
                fn.argtypes = args
            _lib = h
    return _lib


def check(fn: str, status: int) -> None:
    if status != DBS_OK:
        msg = lib().dbs_last_error().decode("utf-8", "replace")
        raise DbsError(fn, status, msg)
