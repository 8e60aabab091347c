"""ctypes loader for libs2attn.so, the C-ABI library.

Loading fails loudly when the library has not been built: there is no
fallback path.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

from .build import LIB_PATH

S2ATTN_OK = 0
S2ATTN_EINVAL = -1
S2ATTN_EUNSUPPORTED = -2
S2ATTN_EHIP = -3
S2ATTN_HEADS_SECOND_HALF = 0
S2ATTN_HEADS_ALTERNATE = 1

_P = ctypes.c_void_p
_I = ctypes.c_int
_D = ctypes.c_double
_S = ctypes.c_size_t

# name -> (restype, argtypes); mirrors include/s2attn.h
SIGNATURES = {
    "s2attn_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P]),
    "s2attn_bwd_workspace_size": (_S, [_I, _I, _I, _I, _I]),
    "s2attn_bwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _S, _P]),
    "s2attn_bwd_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P]),
    "s2attn_bwd_preprocess": (_I, [_P, _P, _P, _I, _I, _I, _I, _P, _S, _P]),
    "s2attn_bwd_dkdv": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _S, _P]),
    "s2attn_bwd_dq": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _S, _P]),
    "s2attn_fwd_rope_workspace_size": (_S, [_I, _I, _I, _I, _I]),
    "s2attn_fwd_rope": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _D, _D, _P, _S, _P]),
    "s2attn_bwd_rope_workspace_size": (_S, [_I, _I, _I, _I, _I]),
    "s2attn_bwd_rope": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _D, _D,
                             _P, _S, _P]),
    "s2attn_fwd_ex": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _D, _D, _P, _S, _P]),
    "s2attn_bwd_ex": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _D, _D,
                           _P, _S, _P]),
    "s2attn_lora_qkv_workspace_size": (_S, [_I, _I]),
    "s2attn_lora_qkv_fwd": (_I, [_P, _I, _I, _P, _P, _P, _I, _I, _P, _P, _P, _P, _P, _P, _I, _D,
                                 _P, _P, _P, _P, _S, _P]),
    "s2attn_lora_qkv_bwd_workspace_size": (_S, [_I, _I, _I, _I, _I]),
    "s2attn_lora_qkv_bwd": (_I, [_P, _I, _I, _P, _P, _P, _I, _I, _P, _P, _P, _P, _P, _P, _I, _D, _P,
                                 _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _S, _P]),
    "s2attn_strerror": (ctypes.c_char_p, [_I]),
    "s2attn_last_error": (ctypes.c_char_p, []),
}

_lib = None


class S2AttnError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"s2attn status {status}: {detail}")


def load(path: str) -> ctypes.CDLL:
    """Open a build of the library at `path` with the ABI's signatures."""
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built; run `python -m grouped_shifted_attention_amd.build` "
            "(or __graft_entry__.build()) first")
    handle = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(handle, name)
        fn.restype = res
        fn.argtypes = args
    return handle


def lib() -> ctypes.CDLL:
    """Load libs2attn.so once; raise if it is missing."""
    global _lib
    if _lib is None:
        _lib = load(LIB_PATH)
    return _lib


@contextlib.contextmanager
def using(handle: ctypes.CDLL):
    """Route the binding's calls to another build of the library (the
    race-check build) for the duration of a with-block."""
    global _lib
    saved = lib()
    _lib = handle
    try:
        yield handle
    finally:
        _lib = saved


def check(status: int) -> None:
    if status != S2ATTN_OK:
        L = lib()
        detail = L.s2attn_last_error().decode() or L.s2attn_strerror(status).decode()
        raise S2AttnError(status, detail)
