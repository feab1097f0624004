"""ctypes declarations of libws (include/ws.h). Loading fails loudly when the
library has not been built: there is no fallback path."""
from __future__ import annotations

import ctypes
import os

from .build import LIB_PATH

WS_OK = 0
WS_ERR_NULL = 1
WS_ERR_SHAPE = 2
WS_ERR_CAPACITY = 3
WS_ERR_ALIGN = 4
WS_ERR_UNSUPPORTED = 5
WS_ERR_WORKSPACE = 6
WS_ERR_HIP = 7

WS_TOKEN_MAJOR = 0
WS_HEAD_MAJOR = 1
WS_MAX_UNITS = 64
WS_SCRATCH_BYTES = 32 << 20


class WsKvCache(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("capacity", ctypes.c_int32),
        ("len", ctypes.c_int32),
    ]


class WsKvSegment(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("n_tok", ctypes.c_int32),
        ("src_heads", ctypes.c_int32),
        ("head_begin", ctypes.c_int32),
        ("layout", ctypes.c_int32),
    ]


WS_MAX_SEGMENTS = 4
_I32P = ctypes.POINTER(ctypes.c_int32)

# name -> (restype, argtypes), exactly as declared in include/ws.h
SIGNATURES = {
    "ws_kv_append": (ctypes.c_int, [ctypes.POINTER(WsKvCache), ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_void_p]),
    "ws_kv_append_segments": (ctypes.c_int, [ctypes.POINTER(WsKvCache), ctypes.POINTER(WsKvSegment),
                                             ctypes.c_int32, ctypes.c_void_p]),
    "ws_attn_default_splits": (ctypes.c_int32, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                ctypes.c_int64]),
    "ws_attn_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                  ctypes.c_int32]),
    "ws_block_causal_attn": (ctypes.c_int, [ctypes.POINTER(WsKvCache), ctypes.c_void_p,
                                            ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_int32, ctypes.c_int32, _I32P, _I32P,
                                            ctypes.c_float, ctypes.c_int32, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "ws_attn_partial": (ctypes.c_int, [ctypes.POINTER(WsKvCache), ctypes.c_void_p, ctypes.c_int32,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                       ctypes.c_int32, _I32P, _I32P, ctypes.c_float, ctypes.c_int32,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                       ctypes.c_void_p]),
    "ws_attn_merge": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                     ctypes.c_void_p]),
    "ws_block_causal_attn_noalloc": (ctypes.c_int, [ctypes.POINTER(WsKvCache), ctypes.c_void_p,
                                                    ctypes.c_int32, ctypes.c_void_p,
                                                    ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                                    _I32P, _I32P, ctypes.c_float, ctypes.c_int32,
                                                    ctypes.c_void_p, ctypes.c_void_p]),
    "ws_fm_euler_step": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                        ctypes.c_float, ctypes.c_void_p]),
    "ws_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "ws_last_error": (ctypes.c_char_p, []),
}

_LIB = None


def lib() -> ctypes.CDLL:
    """The loaded libws with typed entry points (raises if not built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -m cached_block_causal_amd.build)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = handle
    return _LIB


class WsError(RuntimeError):
    def __init__(self, status: int, where: str):
        l = lib()
        self.status = status
        msg = l.ws_status_string(status).decode()
        detail = l.ws_last_error().decode()
        super().__init__(f"{where}: {msg} ({detail})")


def check(status: int, where: str) -> None:
    if status != WS_OK:
        raise WsError(status, where)
