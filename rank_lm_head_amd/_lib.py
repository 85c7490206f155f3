"""ctypes view of liblrhead.so (the C ABI in include/lrhead.h).

Loading fails loudly when the library has not been built: there is no other
implementation of the head in this package.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblrhead.so")

BF16 = 0
FP32 = 1

OK, EINVAL, ERANGE, EDTYPE, EALIGN, EWORKSPACE, EHIP, EDEVICE = 0, -1, -2, -3, -4, -5, -6, -7
K_MAX, R_MAX, D_MAX = 64, 512, 65536
STATIC_SCRATCH_BYTES = 64 << 20   # LRHEAD_STATIC_SCRATCH_MB

_c_i64 = ctypes.c_int64
_vp = ctypes.c_void_p

# name -> (restype, argtypes); the same names as include/lrhead.h
SIGNATURES = {
    "lrhead_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int, _c_i64, _c_i64, _c_i64, _c_i64, ctypes.c_int]),
    "lrhead_create": (ctypes.c_int, [ctypes.POINTER(_vp), ctypes.c_int, _c_i64, _c_i64, _c_i64, _vp, _vp, _vp,
                                     _c_i64, ctypes.c_int, _vp, ctypes.c_size_t]),
    "lrhead_candidates": (ctypes.c_int, [_vp, _vp, _c_i64, ctypes.c_int, _vp, _vp, _vp]),
    "fullhead_logits": (ctypes.c_int, [_vp, _vp, _c_i64, _vp, ctypes.c_int, _vp, _vp]),
    "fullhead_topk": (ctypes.c_int, [_vp, _vp, _c_i64, ctypes.c_int, _vp, _vp, _vp]),
    "lrhead_draft": (ctypes.c_int, [_vp, _vp, _c_i64, ctypes.c_int, _vp, _vp, _vp, _vp]),
    "lrhead_draft_static": (ctypes.c_int, [ctypes.c_int, _c_i64, _c_i64, _c_i64, _vp, _vp, _vp, _vp, _c_i64,
                                           ctypes.c_int, _vp, _vp, _vp, _vp]),
    "lrhead_branch": (ctypes.c_int, [_vp, _vp, _vp, _c_i64, ctypes.c_int, ctypes.c_int, _vp, _vp, _vp, _vp, _vp]),
    "lrhead_factor_workspace_bytes": (ctypes.c_size_t, [_c_i64, _c_i64, ctypes.c_int]),
    "lrhead_factor": (ctypes.c_int, [_vp, _c_i64, _c_i64, ctypes.c_int, ctypes.c_int, _vp, _vp, _vp, _vp,
                                     ctypes.c_size_t, _vp]),
    "lrhead_set_stage_events": (ctypes.c_int, [_vp, _vp, _vp]),
    "lrhead_destroy": (None, [_vp]),
    "lrhead_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "lrhead_last_error": (ctypes.c_char_p, []),
}

_lib = None


class LrheadError(RuntimeError):
    def __init__(self, code: int, where: str):
        lib = load()
        detail = lib.lrhead_last_error().decode(errors="replace")
        text = lib.lrhead_strerror(code).decode()
        super().__init__(f"{where}: {text} ({code}): {detail}")
        self.code = code


def load():
    """The loaded library, with argument and return types set."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python -m rank_lm_head_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def check(code: int, where: str) -> None:
    if code != OK:
        raise LrheadError(code, where)
