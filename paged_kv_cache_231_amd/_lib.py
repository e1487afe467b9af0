"""ctypes loader of libpkv.so and the signatures of include/pkv.h.

Loading fails loudly: if the library is missing it is built with hipcc; if
that fails, or the library cannot be loaded, an exception is raised.  There
is no fallback implementation.
"""

from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpkv.so")

STATUS = {0: "OK", 1: "EINVAL", 2: "ESHAPE", 3: "ERANGE", 4: "EDEVICE", 5: "EWORKSPACE", 6: "EHIP"}

_u32 = ctypes.c_uint32
_p = ctypes.c_void_p
_pu32 = ctypes.POINTER(ctypes.c_uint32)
_size = ctypes.c_size_t
_f = ctypes.c_float
_i = ctypes.c_int

class AppendReport(ctypes.Structure):
    """pkv_append_report."""
    _fields_ = [("key_copied", ctypes.c_uint32), ("value_copied", ctypes.c_uint32),
                ("copied_bytes", ctypes.c_uint64)]


# name: (restype, argtypes) for every function of include/pkv.h
SIGNATURES = {
    "pkv_plan_encode": (_i, [_u32, _pu32, _u32, _pu32, _pu32, _u32, _pu32, _u32, _u32, _pu32,
                             ctypes.POINTER(_size)]),
    "pkv_plan_validate": (_i, [_pu32, _size]),
    "pkv_plan_validate_writes": (_i, [_pu32, _size]),
    "pkv_plan_create": (_i, [_pu32, _size, _p, ctypes.POINTER(_p)]),
    "pkv_plan_rebind_async": (_i, [_p, _p, _size, _p]),
    "pkv_plan_set_word_async": (_i, [_p, _size, _u32, _p]),
    "pkv_plan_header": (_i, [_p, _pu32]),
    "pkv_plan_device_words": (_p, [_p]),
    "pkv_plan_destroy": (None, [_p]),
    "pkv_workspace_create": (_i, [_u32, _u32, _u32, _u32, _p, ctypes.POINTER(_p)]),
    "pkv_workspace_create_balanced": (_i, [_u32, _u32, _u32, _p, ctypes.POINTER(_p)]),
    "pkv_workspace_splits": (_u32, [_p]),
    "pkv_workspace_destroy": (None, [_p]),
    "pkv_suggest_splits": (_u32, [_p, _u32, _u32, _u32]),
    "pkv_tune_splits": (_i, [_p, _i, _p, _p, _p, _p, _u32, _u32, _u32, _u32, _f, _i, _u32, _p,
                             ctypes.POINTER(_u32)]),
    "pkv_tune_splits_mla": (_i, [_p, _i, _p, _p, _p, _p, _p, _u32, _u32, _u32, _f, _i, _u32, _p,
                                 ctypes.POINTER(_u32)]),
    "pkv_attention": (_i, [_p, _i, _p, _p, _p, _p, _u32, _u32, _u32, _u32, _f, _i, _p, _p]),
    "pkv_attention_window": (_i, [_p, _i, _p, _p, _p, _p, _u32, _u32, _u32, _u32, _f, _i, _u32,
                                  _p, _p]),
    "pkv_attention_noalloc": (_i, [_p, _i, _p, _p, _p, _p, _u32, _u32, _u32, _u32, _f, _i, _p]),
    "pkv_attention_fp8": (_i, [_p, _i, _p, _p, _p, _p, _u32, _u32, _u32, _u32, _f, _f, _f, _i,
                               _u32, _p, _p]),
    "pkv_mla": (_i, [_p, _i, _p, _p, _p, _p, _p, _u32, _u32, _u32, _f, _i, _p, _p]),
    "pkv_append": (_i, [_p, _i, _p, _p, _p, _p, _p, _p, _u32, _u32, _u32,
                        ctypes.POINTER(AppendReport), _p]),
    "pkv_plan_timing": (_i, [_p, _i]),
    "pkv_plan_timing_select": (_i, [_p, _u32]),
    "pkv_plan_timing_read": (_i, [_p, _i, ctypes.POINTER(_u32), ctypes.POINTER(ctypes.c_double)]),
    "pkv_last_error": (ctypes.c_char_p, []),
    "pkv_version": (ctypes.c_char_p, []),
}

_lock = threading.Lock()
_lib = None


class PKVError(RuntimeError):
    """A pkv_status other than PKV_OK, with the library's static message."""

    def __init__(self, code: str, message: str):
        super().__init__(f"{code}: {message}")
        self.code = code
        self.message = message


def lib() -> ctypes.CDLL:
    """The loaded library (built first if it does not exist yet)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                from . import build as _build
                _build.build()
            handle = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(handle, name)
                fn.restype = res
                fn.argtypes = args
            _lib = handle
        return _lib


def check(status: int) -> None:
    if status != 0:
        msg = lib().pkv_last_error().decode()
        raise PKVError(STATUS.get(status, f"E{status}"), msg)
