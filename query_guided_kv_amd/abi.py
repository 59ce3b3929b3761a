"""ctypes declarations of libkvsel's C ABI (``include/kvsel.h``).

Plain ctypes, no torch: the structs, the status and enum values, every
exported signature, and :func:`load`.  :mod:`query_guided_kv_amd.kvsel` builds
the tensor-level binding on top of this module.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvsel.so")

# status codes
OK, ERR_NULL, ERR_SHAPE, ERR_DTYPE, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, -1, -2, -3, -4, -5, -6
# element types, RoPE pairings, aggregation signals
BF16, FP32 = 0, 1
ROPE = {"half": 0, "interleaved": 1}
SIGNAL = {"mass": 0, "vnorm": 1}


class Cache(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("N", ctypes.c_int64), ("H", ctypes.c_int64),
                ("D", ctypes.c_int64), ("stride_b", ctypes.c_int64),
                ("stride_n", ctypes.c_int64), ("dtype", ctypes.c_int32)]


class Segment(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("kc", Cache)]


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_F = ctypes.c_float
_D = ctypes.c_double
_SZ = ctypes.c_size_t

SIGNATURES = {
    "kvsel_reposition": (ctypes.c_int, [_P, _P, Cache, _I64, _P, _I32, _D, _I32, _P]),
    "kvsel_score": (ctypes.c_int, [_P, _I64, _I64, _P, Cache, _F, _I64, _P, _P, _P, _P, _SZ, _P]),
    "kvsel_score_workspace": (_SZ, [_I64, _I64, _I64, _I64, _I64, _I32, _I32]),
    "kvsel_score_reposition": (ctypes.c_int, [_P, _I64, _I64, _P, _P, Cache, _F, _I64, _I64, _P,
                                              _I32, _D, _I32, _P, _P, _P, _P, _SZ, _P]),
    "kvsel_score_reposition_workspace": (_SZ, [_I64, _I64, Cache, _I64, _I64, _I32, _I32, _I32]),
    "kvsel_aggregate": (ctypes.c_int, [_P, _I64, _I64, _P, _P, Cache, _F, _P, _P, _P, _I32, _I64,
                                       _I64, _P, _I32, _P, _SZ, _P]),
    "kvsel_score_units": (ctypes.c_int, [_P, _I64, _I64, _P, Cache, _F, _I64, _P, _I64, _P, _I32,
                                         _D, _I32, _P, _P, _P, _P, _SZ, _P]),
    "kvsel_score_units_workspace": (_SZ, [_I64, _I64, Cache, _I64, _I64, _I32, _I32]),
    "kvsel_take": (ctypes.c_int, [_P, _I64, _I64, _P, _I64, _P, _P]),
    "kvsel_order": (ctypes.c_int, [_P, _I64, _I64, _P, _I64, _I32, _P, _P, _P]),
    "kvsel_index_attn": (ctypes.c_int, [_P, _I64, _I64, _F, _P, _P, Cache, _P, _P, _P, _P]),
    "kvsel_unit_fractions": (ctypes.c_int, [_P, _I64, _I64, _I64, _I64, _P, _P]),
    "kvsel_slot_starts": (ctypes.c_int, [_P, _I64, _I64, _I64, _I64, _I64, _P, _P]),
    "kvsel_aggregate_workspace": (_SZ, [_I64, _I64, _I64, _I64, _I64, _I32, _I32]),
    "kvsel_topk": (ctypes.c_int, [_P, _I64, _I64, _I64, _P, _P, _P]),
    "kvsel_gather": (ctypes.c_int, [_P, _P, Cache, _I64, _P, _I64, _I64, _P, _I64, _D, _I32, _P,
                                    _P, ctypes.POINTER(Cache), _P, _P, _P]),
    "kvsel_decode_attn": (ctypes.c_int, [_P, _I64, _I64, _F, ctypes.POINTER(Segment), _I32, _P,
                                         _P, _P, _SZ, _P]),
    "kvsel_decode_workspace": (_SZ, [_I64, _I64, ctypes.POINTER(Segment), _I32]),
    "kvsel_gather_decode": (ctypes.c_int, [_P, _I64, _I64, _F, _P, _P, Cache, _I64, _P, _I64, _I64,
                                           _P, _P, ctypes.POINTER(Segment), _I32, _P, _P, _P, _SZ,
                                           _P]),
    "kvsel_gather_decode_workspace": (_SZ, [_I64, _I64, Cache, _I64, _I64, ctypes.POINTER(Segment),
                                            _I32]),
    "kvsel_gather_decode_noalloc": (ctypes.c_int, [_P, _I64, _I64, _F, _P, _P, Cache, _I64, _P,
                                                   _I64, _I64, _P, _P, ctypes.POINTER(Segment),
                                                   _I32, _P, _P, _P]),
    "kvsel_noalloc_scratch_bytes": (_SZ, []),
    "kvsel_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "kvsel_last_error": (ctypes.c_char_p, []),
    "kvsel_version": (ctypes.c_int, []),
}

_lib: Optional[ctypes.CDLL] = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libkvsel.so (built in-tree by ``query_guided_kv_amd.build``); any
    other path (another build of the same sources) is loaded afresh."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m query_guided_kv_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path == LIB_PATH:
        _lib = lib
    return lib
