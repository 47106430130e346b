"""ctypes view of libmars.so: symbol loading and signatures only.

The library must exist (build it with `python -m block_masked_causal_amd.build`);
there is no fallback implementation of any kind.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmars.so")

MARS_OK = 0
MARS_ERR_NULL = -1
MARS_ERR_SHAPE = -2
MARS_ERR_DTYPE = -3
MARS_ERR_UNSUPPORTED = -4
MARS_ERR_ALIGN = -5
MARS_ERR_WORKSPACE = -6
MARS_ERR_LAUNCH = -7

MARS_F32 = 0
MARS_BF16 = 1

NOALLOC_SCRATCH_BYTES = 16 << 20  # MARS_NOALLOC_SCRATCH_BYTES

STATUS_CACHE_OVERFLOW = 1
STATUS_BAD_PAGE = 2
STATUS_NONFINITE = 4

_i32 = ctypes.c_int32
_p = ctypes.c_void_p
_f = ctypes.c_float
_sz = ctypes.c_size_t

SIGNATURES = {
    "mars_attn_two_stream": (ctypes.c_int, [_p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32,
                                            _i32, _i32, _f, _i32, _p]),
    "mars_attn_causal": (ctypes.c_int, [_p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32,
                                        _f, _p]),
    "mars_attn_block_decode_rows": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _i32,
                                                   _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                                   _i32, _f, _p, _sz, _p, _p]),
    "mars_block_sync_accept": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32,
                                              _i32, _p, _p]),
    "mars_block_freeze": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32,
                                         _i32, _i32, _i32, _i32, _i32, _p, _p]),
    "mars_kv_append": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32,
                                      _i32, _i32, _p, _p]),
    "mars_attn_two_stream_bwd": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _i32, _i32,
                                                _i32, _i32, _i32, _i32, _i32, _f, _i32, _p, _sz,
                                                _p]),
    "mars_attn_two_stream_bwd_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "mars_attn_block_decode": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32,
                                              _i32, _i32, _i32, _i32, _i32, _i32, _f, _p, _sz,
                                              _p, _p]),
    "mars_decode_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "mars_lmhead_confidence": (ctypes.c_int, [_p, _p, _p, _i32, _i32, _i32, _p, _p, _p, _sz,
                                              _p, _p]),
    "mars_lmhead_workspace_bytes": (_sz, [_i32, _i32]),
    "mars_lmhead_confidence_noalloc": (ctypes.c_int, [_p, _p, _p, _i32, _i32, _i32, _p, _p, _p,
                                                      _p]),
    "mars_lmhead_packed_bytes": (_sz, [_i32, _i32]),
    "mars_lmhead_pack": (ctypes.c_int, [_p, _p, _i32, _i32, _p]),
    "mars_lmhead_confidence_packed": (ctypes.c_int, [_p, _p, _p, _i32, _i32, _i32, _p, _p, _p,
                                                     _sz, _p, _p]),
    "mars_accept_commit": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _i32,
                                          _i32, _i32, _i32, _i32, _i32, _i32, _i32, _p, _p]),
    "mars_accept_commit_layers": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                                                 _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                                 _i32, _p, _p]),
    "mars_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "mars_version": (ctypes.c_int, []),
}

_lib = None


class MarsError(RuntimeError):
    def __init__(self, fn: str, code: int):
        self.code = code
        super().__init__(f"{fn} failed with code {code}: {strerror(code)}")


def lib() -> ctypes.CDLL:
    """Load libmars.so once; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m block_masked_causal_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().mars_strerror(code).decode()


def check(fn: str, code: int) -> None:
    if code != MARS_OK:
        raise MarsError(fn, code)
