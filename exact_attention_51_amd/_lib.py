"""ctypes loader for libfa.so and the raw C-ABI signatures (include/fa.h)."""

from __future__ import annotations

import ctypes
import os

from .build import LIB_PATH

FA_OK = 0
FA_ERR_INVALID_ARG = -1
FA_ERR_UNSUPPORTED = -2
FA_ERR_LAUNCH = -3
FA_FWD_KV_NOALLOC_MAX_BYTES = 64 << 20  # include/fa.h

# name -> (restype, argtypes); must match include/fa.h exactly.
_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
SIGNATURES = {
    "fa_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P]),
    "fa_fwd_f32": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P]),
    "fa_fwd_kv": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _I, _P, ctypes.c_size_t, _P]),
    "fa_fwd_kv_noalloc": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _I, _P]),
    "fa_fwd_kv_splits": (_I, [_I, _I, _I, _I, _I, _I]),
    "fa_fwd_sparse": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P, _I, _P]),
    "fa_fwd_kv_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I, _I]),
    "fa_bwd_dq": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P]),
    "fa_bwd_dkdv": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P]),
    "fa_strerror": (ctypes.c_char_p, [_I]),
    "fa_version": (_I, []),
}

_lib = None


class FAError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed with code {code}: {msg}")
        self.code = code


def load(path: str | None = None) -> ctypes.CDLL:
    """Load libfa.so (built in-tree by build.py).  Raises if it is missing."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or os.environ.get("FA_LIB", LIB_PATH)
    if not os.path.exists(p):
        raise ImportError(f"{p} is not built; run `python -m exact_attention_51_amd.build` first")
    lib = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def check(fn: str, code: int) -> None:
    if code != FA_OK:
        raise FAError(fn, code, load().fa_strerror(code).decode())
