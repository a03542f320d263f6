"""ctypes loader for libattn.so.  Raises if the library is missing: there is no fallback path."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libattn.so")

ATTN_OK, ATTN_ERR_INVALID, ATTN_ERR_UNSUPPORTED, ATTN_ERR_WORKSPACE, ATTN_ERR_HIP = range(5)
ATTN_F32, ATTN_BF16 = 0, 1
SKIP_TILE = 32
NOALLOC_SCRATCH_BYTES = 64 << 20  # ATTN_NOALLOC_SCRATCH_BYTES

# name -> (restype, argtypes), mirroring include/attn.h
_P, _I, _F, _Z = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
SIGNATURES = {
    "attn_prefill_varlen": (ctypes.c_int, [_I, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _F, _P, _P, _P,
                                           _I, _P]),
    "attn_decode_paged_workspace_size": (_Z, [_I, _I, _I, _I]),
    "attn_decode_paged": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _F, _I, _P, _Z, _P, _P,
                                         _P, _I, _P]),
    "attn_decode_paged_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _F, _I, _P, _P,
                                                 _P, _I, _P]),
    "attn_decode_paged_qdq": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _F, _F, _F, _P,
                                             _P, _P, _I, _P]),
    "attn_decode_paged_multi_workspace_size": (_Z, [_I, _I, _I, _I, _I, _I]),
    "attn_decode_paged_multi": (ctypes.c_int, [_P, _P, _I, _I, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _F,
                                               _I, _P, _Z, _P, _P, _P, _I, _P]),
    "attn_smallseq_cross": (ctypes.c_int, [_P, _P, _P, _P, _I, _I, _I, _I, _F, _P, _P, _P, _P]),
    "attn_smallseq_cross_backward": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _P, _P, _P, _P]),
    "attn_prefill_varlen_backward_workspace_size": (_Z, [_I, _I, _I]),
    "attn_prefill_varlen_backward": (ctypes.c_int, [_I, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F,
                                                    _I, _P, _P, _P, _P, _Z, _P]),
    "attn_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "attn_last_error_message": (ctypes.c_char_p, []),
}

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


def load():
    """Loads libattn.so once and declares every exported signature."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python -m paged_skip_softmax_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        _lib = lib
    return _lib


def check(status: int) -> None:
    if status != ATTN_OK:
        lib = load()
        raise AttnError(status, lib.attn_last_error_message().decode() or lib.attn_status_string(status).decode())
