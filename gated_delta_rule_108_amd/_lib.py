"""ctypes view of libkda.so (the C ABI declared in include/kda.h).

Loading never falls back to anything: if the library is missing or does not
export a symbol, the import of the binding fails with an explicit error.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkda.so")

KDA_OK = 0
KDA_ERR_NULL = -1
KDA_ERR_SHAPE = -2
KDA_ERR_UNSUPPORTED = -3
KDA_ERR_ALIGN = -4
KDA_ERR_ALIAS = -5
KDA_ERR_WORKSPACE = -6
KDA_ERR_DEVICE = -7
KDA_ERR_HIP = -8
KDA_ERR_SCRATCH = -9

KDA_F32 = 0
KDA_BF16 = 1

KDA_QK_AS_GIVEN = 0
KDA_QK_L2 = 1
KDA_QK_SILU_L2 = 2

# (name, restype, argtypes) for every entry point of include/kda.h
_vp, _i, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
SIGNATURES = {
    "kda_prefill_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "kda_prefill_chunked": (ctypes.c_int32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                             _i, _i, _i, _i, _i, _i, _i, _vp, _sz, _vp]),
    "kda_decode_step": (ctypes.c_int32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                         _i, _i, _i, _i, _i, _vp]),
    "kda_prefill_chunked_noalloc": (ctypes.c_int32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                                     _i, _i, _i, _i, _i, _i, _i, _vp]),
    "kda_prefill_chunked_logits": (ctypes.c_int32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                                    _i, _i, _i, _i, _i, _i, _i, _i, _vp, _sz,
                                                    _vp]),
    "kda_decode_step_logits": (ctypes.c_int32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                                _i, _i, _i, _i, _i, _i, _vp]),
    "kda_gdn_prefill_chunked": (ctypes.c_int32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                                 _i, _i, _i, _i, _i, _i, _i, _vp, _sz, _vp]),
    "kda_gdn_decode_step": (ctypes.c_int32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                             _i, _i, _i, _i, _i, _vp]),
    "kda_decode_step_backward": (ctypes.c_int32, [_vp] * 14 + [_i, _i, _i, _i, _i, _vp]),
    "kda_prefill_backward_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "kda_prefill_backward": (ctypes.c_int32, [_vp] * 14 + [_i] * 6 + [_vp, _sz, _vp]),
    "kda_gdn_prefill_backward": (ctypes.c_int32, [_vp] * 14 + [_i] * 6 + [_vp, _sz, _vp]),
    "kda_prefill_backward_chunked_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "kda_prefill_backward_chunked": (ctypes.c_int32, [_vp] * 14 + [_i] * 6 + [_vp, _sz, _vp]),
    "kda_gdn_decode_step_backward": (ctypes.c_int32, [_vp] * 14 + [_i, _i, _i, _i, _i, _vp]),
    "kda_prologue_forward": (ctypes.c_int32, [_vp] * 8 + [_i] * 4 + [_vp]),
    "kda_prologue_backward": (ctypes.c_int32, [_vp] * 12 + [_i] * 4 + [_vp]),
    "kda_status_string": (ctypes.c_char_p, [ctypes.c_int32]),
}

_lib = None


class KDAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_string(status)})")


def load(path: str = LIB_PATH):
    """Load libkda.so once and attach the ABI signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with __graft_entry__.build() "
                          "(hipcc, gfx950); there is no fallback implementation")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)  # AttributeError if the symbol is absent
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().kda_status_string(status).decode()
