"""ctypes declarations of the C ABI in include/mla.h (argument marshalling only)."""

from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int32, c_int64, c_void_p

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmla.so")
HOST_LIB_PATH = os.path.join(PKG, "libmla_host.so")

_i32p = POINTER(c_int32)
_i64p = POINTER(c_int64)
_f32p = POINTER(c_float)

# Every function include/mla.h declares, with (restype, argtypes).
SIGNATURES = {
    "mla_plan_create": (c_int32, [POINTER(c_void_p), c_int32, c_int32, c_int32, c_int32, c_int32]),
    "mla_plan_reserve": (c_int32, [c_void_p, c_int32, c_int64, c_int64]),
    "mla_plan": (c_int32, [c_void_p, _i32p, _i32p, _i32p, _i32p, c_int32, c_int32, c_float,
                           c_int64, c_void_p]),
    "mla_run": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "mla_run_fp8": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_float, c_void_p,
                              c_void_p, c_void_p]),
    "mla_append_kv": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "mla_append_kv_fp8": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_float, c_void_p]),
    "mla_absorb_query": (c_int32, [c_void_p, c_void_p, c_void_p, c_int64, c_int32, c_void_p]),
    "mla_up_project": (c_int32, [c_void_p, c_void_p, c_void_p, c_int64, c_int32, c_void_p]),
    "mla_merge_state": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                  c_int64, c_int32, c_void_p]),
    "mla_run_noalloc": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int64,
                                  c_int64, c_int32, c_float, c_int64, c_int32, c_int32, c_int32,
                                  c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "mla_plan_destroy": (None, [c_void_p]),
    "mla_plan_stats": (c_int32, [c_void_p, _i32p, _i64p, _i64p, _i64p]),
    "mla_status_str": (c_char_p, [c_int32]),
    "mla_last_error": (c_char_p, []),
    "mla_schedule_build": (c_int32, [POINTER(c_void_p), _i32p, _i32p, _i32p, _i32p, c_int32,
                                     c_int32, c_int32, c_int64, c_int32, c_int32]),
    "mla_schedule_sizes": (None, [c_void_p, _i32p, _i64p, _i64p, _i64p]),
    "mla_schedule_copy": (None, [c_void_p, _i32p, _i32p, _i32p]),
    "mla_schedule_append_rows": (c_int32, [c_void_p, _i32p]),
    "mla_schedule_destroy": (None, [c_void_p]),
}

HOST_ONLY = ("mla_status_str", "mla_last_error", "mla_schedule_build", "mla_schedule_sizes",
             "mla_schedule_copy", "mla_schedule_append_rows", "mla_schedule_destroy")

_cache = {}


def load(path: str = LIB_PATH, host_only: bool = False) -> ctypes.CDLL:
    """Load a built library and declare its functions.  Raises if missing."""
    key = (path, host_only)
    if key in _cache:
        return _cache[key]
    if not os.path.exists(path):
        raise RuntimeError(
            f"native library {path} is not built; run `python -m paged_mla_attention_amd.build`")
    lib = ctypes.CDLL(path)
    names = HOST_ONLY if host_only else SIGNATURES
    for name in names:
        res, args = SIGNATURES[name]
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _cache[key] = lib
    return lib


class MLAError(RuntimeError):
    def __init__(self, lib, status: int):
        self.status = int(status)
        msg = lib.mla_last_error().decode()
        name = lib.mla_status_str(status).decode()
        super().__init__(f"{name} ({status}): {msg}")


def check(lib, status: int) -> None:
    if status != 0:
        raise MLAError(lib, status)
