"""ctypes view of libpagedkv.so (declared in include/paged_kv.h).

torch is imported first so that its HIP runtime is already in the process: the library then binds to
that same runtime (both carry the soname libamdhip64.so.7), and the device pointers and streams torch
hands out are valid in it.  There is no fallback: if the library is missing, loading fails loudly.
"""

from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (must precede the library load, see above)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagedkv.so")

PKV_OK = 0
PKV_ERR_INVALID_ARG = -1
PKV_ERR_UNSUPPORTED = -2
PKV_ERR_WORKSPACE = -3
PKV_ERR_HIP = -4
PKV_ERR_NO_BLOCKS = -5
PKV_FP32 = 0
PKV_BF16 = 1
PKV_NOALLOC_SCRATCH_BYTES = 33554432

STATUS_NAMES = {
    PKV_OK: "PKV_OK",
    PKV_ERR_INVALID_ARG: "PKV_ERR_INVALID_ARG",
    PKV_ERR_UNSUPPORTED: "PKV_ERR_UNSUPPORTED",
    PKV_ERR_WORKSPACE: "PKV_ERR_WORKSPACE",
    PKV_ERR_HIP: "PKV_ERR_HIP",
    PKV_ERR_NO_BLOCKS: "PKV_ERR_NO_BLOCKS",
}

# Every symbol include/paged_kv.h declares, with its ctypes signature.
_c = ctypes
_vp, _i32, _i64, _sz, _f32 = _c.c_void_p, _c.c_int32, _c.c_int64, _c.c_size_t, _c.c_float
_u64 = _c.c_uint64
SIGNATURES = {
    "paged_kv_abi_version": (_c.c_int, []),
    "paged_kv_last_error": (_c.c_char_p, []),
    "paged_kv_write": (_c.c_int, [_vp, _vp, _vp, _i64, _vp, _vp, _i64, _i32, _i64, _i32, _i32, _i32, _vp]),
    "paged_attention_workspace_size": (_sz, [_i32, _i64, _i32, _i32, _i32, _i32, _i32]),
    "paged_attention_forward": (_c.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32, _i64, _i32,
                                           _i32, _i32, _i32, _i64, _i64, _f32, _i32, _i32, _vp, _sz,
                                           _vp]),
    "paged_attention_write_forward": (_c.c_int, [_vp, _vp, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp,
                                                 _i32, _i64, _i32, _i32, _i32, _i32, _i64, _i64, _f32, _i32,
                                                 _i32, _vp, _sz, _vp]),
    "paged_attention_run": (_c.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32, _i64, _i32,
                                       _i32, _i32, _i32, _i64, _i64, _f32, _i32, _i32, _vp, _sz, _vp]),
    "paged_attention_forward_noalloc": (_c.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32, _i64, _i32,
                                                   _i32, _i32, _i32, _i64, _i64, _f32, _i32, _i32, _vp]),
    "paged_attention_prefix_workspace_size": (_sz, [_i32, _i64, _i32, _i32, _i32, _i32]),
    "paged_attention_forward_prefix": (_c.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32, _i64,
                                                  _i32, _i32, _i32, _i32, _i64, _i64, _f32, _i32, _i32,
                                                  _i32, _i32, _vp, _sz, _vp]),
    "paged_attention_run_prefix": (_c.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32, _i64,
                                              _i32, _i32, _i32, _i32, _i64, _i64, _f32, _i32, _i32,
                                              _i32, _i32, _vp, _sz, _vp]),
    "paged_attention_set_tuning": (_c.c_int, [_i32, _i32, _i32]),
    "paged_attention_set_profile_events": (_c.c_int, [_vp, _vp]),
    "paged_kv_copy_blocks": (_c.c_int, [_vp, _vp, _i64, _i32, _i64, _i32, _i32, _i32, _vp, _vp, _i32, _vp]),
    "pkv_cm_create": (_vp, [_i32, _i32]),
    "pkv_cm_destroy": (None, [_vp]),
    "pkv_cm_num_free": (_i32, [_vp]),
    "pkv_cm_seq_len": (_i32, [_vp, _i64]),
    "pkv_cm_append": (_c.c_int, [_vp, _i64, _i32, _vp, _vp]),
    "pkv_cm_free": (_c.c_int, [_vp, _i64]),
    "pkv_cm_fork": (_c.c_int, [_vp, _i64, _i64]),
    "pkv_cm_add_prefix": (_c.c_int, [_vp, _u64, _i64, _i32]),
    "pkv_cm_attach_prefix": (_c.c_int, [_vp, _u64, _i64, _vp]),
    "pkv_cm_drop_prefix": (_c.c_int, [_vp, _u64]),
    "pkv_cm_build_tables": (_c.c_int, [_vp, _vp, _i32, _i32, _vp, _vp]),
}

_LIB = None


class PagedKVError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded library (loaded on first use)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; build it with `python -m paged_kv_cache_229_amd.build` "
                "(or __graft_entry__.build()) before using the paged KV-cache ops")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = handle
    return _LIB


def check(status: int) -> None:
    if status != PKV_OK:
        raise PagedKVError(status, lib().paged_kv_last_error().decode(errors="replace"))
