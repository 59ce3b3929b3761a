"""Python binding of libkvsel (ctypes).  Argument marshalling only.

Each function mirrors one C entry point of ``include/kvsel.h``: it takes torch
tensors that live on the GPU, allocates outputs and workspace with torch's
caching allocator, passes raw device pointers and the current HIP stream, and
raises :class:`KvselError` on a negative status.  All computation happens in
the library's kernels; there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvsel.so")

BF16, FP32 = 0, 1
ROPE = {"half": 0, "interleaved": 1}
SIGNAL = {"mass": 0, "vnorm": 1}


class KvselError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"kvsel status {status}: {msg}")
        self.status = status


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

_SIGNATURES = {
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
    "kvsel_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "kvsel_last_error": (ctypes.c_char_p, []),
    "kvsel_version": (ctypes.c_int, []),
}

_lib: Optional[ctypes.CDLL] = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libkvsel.so (built in-tree by ``query_guided_kv_amd.build``)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m query_guided_kv_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path == LIB_PATH:
        _lib = lib
    return lib


def _check(rc: int) -> None:
    if rc != 0:
        lib = load()
        raise KvselError(rc, f"{lib.kvsel_status_str(rc).decode()}: {lib.kvsel_last_error().decode()}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return FP32
    raise KvselError(-3, f"unsupported dtype {t.dtype}")


def cache_desc(t: torch.Tensor) -> Cache:
    """Descriptor of a [B][N][H][D] tensor whose [H][D] block is contiguous."""
    if t.dim() != 4:
        raise KvselError(-2, f"cache must be [B][N][H][D], got {tuple(t.shape)}")
    B, N, H, D = t.shape
    if t.stride(3) != 1 or t.stride(2) != D:
        raise KvselError(-4, "cache rows must hold contiguous [H][D]")
    return Cache(B, N, H, D, t.stride(0), t.stride(1), dtype_code(t))


def _empty(shape, dev, dtype=torch.float32):
    return torch.empty(shape, dtype=dtype, device=dev)


def _workspace(nbytes: int, dev) -> Optional[torch.Tensor]:
    return torch.empty(max(1, (nbytes + 255) // 256 * 256), dtype=torch.uint8, device=dev) if nbytes else None


# ---------------------------------------------------------------------------
# the six calls
# ---------------------------------------------------------------------------

def reposition(k: torch.Tensor, delta: torch.Tensor, unit_len: int,
               out: Optional[torch.Tensor] = None, rope_base: float = 10000.0,
               style: str = "half") -> torch.Tensor:
    """kvsel_reposition: rotate every row of unit u by delta[u] positions.
    ``delta``: int64 [M] or [B][M] on the device.  ``out`` may be ``k`` (in place)."""
    lib = load()
    out = torch.empty_like(k) if out is None else out
    if out.shape != k.shape or out.stride() != k.stride():
        raise KvselError(-2, "out must match k in shape and strides")
    per = 1 if delta.dim() == 2 else 0
    _check(lib.kvsel_reposition(_ptr(k), _ptr(out), cache_desc(k), unit_len, _ptr(delta), per,
                                rope_base, ROPE[style], _stream(k.device)))
    return out


def score(q: torch.Tensor, k: torch.Tensor, unit_len: int, scale: Optional[float] = None,
          row_stats: bool = True, partials: bool = True):
    """kvsel_score -> (row_max, row_sum, part); entries not requested are None."""
    lib = load()
    B, T, Hq, D = q.shape
    N = k.shape[1]
    scale = 1.0 / D ** 0.5 if scale is None else scale
    dev = k.device
    rm = _empty((B, Hq, T), dev) if row_stats else None
    rs = _empty((B, Hq, T), dev) if row_stats else None
    part = _empty((B, Hq, T, N // unit_len, 2), dev) if partials else None
    need = lib.kvsel_score_workspace(B, N, Hq, T, unit_len, int(row_stats), int(partials))
    ws = _workspace(need, dev)
    _check(lib.kvsel_score(_ptr(q), T, Hq, _ptr(k), cache_desc(k), scale, unit_len, _ptr(rm),
                           _ptr(rs), _ptr(part), _ptr(ws), need, _stream(dev)))
    return rm, rs, part


def score_reposition(q: torch.Tensor, k: torch.Tensor, delta: torch.Tensor, rot_unit_len: int,
                     unit_len: int, k_out: Optional[torch.Tensor] = None,
                     scale: Optional[float] = None, row_stats: bool = True,
                     partials: bool = True, rope_base: float = 10000.0, style: str = "half"):
    """kvsel_score_reposition -> (row_max, row_sum, part) of the keys rotated by
    delta[u] per unit of ``rot_unit_len`` rows; ``k_out`` (same shape and strides
    as ``k``) receives the re-positioned keys when given."""
    lib = load()
    B, T, Hq, D = q.shape
    N = k.shape[1]
    scale = 1.0 / D ** 0.5 if scale is None else scale
    dev = k.device
    if k_out is not None and (k_out.shape != k.shape or k_out.stride() != k.stride()):
        raise KvselError(-2, "k_out must match k in shape and strides")
    rm = _empty((B, Hq, T), dev) if row_stats else None
    rs = _empty((B, Hq, T), dev) if row_stats else None
    part = _empty((B, Hq, T, N // unit_len, 2), dev) if partials else None
    kc = cache_desc(k)
    need = lib.kvsel_score_reposition_workspace(T, Hq, kc, unit_len, rot_unit_len,
                                                int(row_stats), int(partials),
                                                int(k_out is not None))
    ws = _workspace(need, dev)
    per = 1 if delta.dim() == 2 else 0
    _check(lib.kvsel_score_reposition(_ptr(q), T, Hq, _ptr(k), _ptr(k_out), kc, scale, unit_len,
                                      rot_unit_len, _ptr(delta), per, rope_base, ROPE[style],
                                      _ptr(rm), _ptr(rs), _ptr(part), _ptr(ws), need,
                                      _stream(dev)))
    return rm, rs, part


def score_units(q: torch.Tensor, k: torch.Tensor, units: torch.Tensor, unit_len: int,
                delta: Optional[torch.Tensor] = None, scale: Optional[float] = None,
                row_stats: bool = True, partials: bool = True, rope_base: float = 10000.0,
                style: str = "half"):
    """kvsel_score_units -> (row_max, row_sum, part) of each instance's query
    block against the listed units of its cache (``units`` int32 [B][n]), unit
    j re-positioned by ``delta[j]`` (int64 [n] or [B][n]) when given.  ``k``
    may be a strided view, e.g. one layer of a [R][L][N][H][D] store."""
    lib = load()
    B, T, Hq, D = q.shape
    n = units.shape[1]
    if units.dtype != torch.int32 or units.dim() != 2 or units.shape[0] != k.shape[0] \
            or not units.is_contiguous():
        raise KvselError(-2, "units must be contiguous int32 [B][n_units]")
    scale = 1.0 / D ** 0.5 if scale is None else scale
    dev = k.device
    rm = _empty((B, Hq, T), dev) if row_stats else None
    rs = _empty((B, Hq, T), dev) if row_stats else None
    part = _empty((B, Hq, T, n, 2), dev) if partials else None
    kc = cache_desc(k)
    need = lib.kvsel_score_units_workspace(T, Hq, kc, unit_len, n, int(row_stats), int(partials))
    ws = _workspace(need, dev)
    per = 1 if delta is not None and delta.dim() == 2 else 0
    _check(lib.kvsel_score_units(_ptr(q), T, Hq, _ptr(k), kc, scale, unit_len, _ptr(units), n,
                                 _ptr(delta), per, rope_base, ROPE[style], _ptr(rm), _ptr(rs),
                                 _ptr(part), _ptr(ws), need, _stream(dev)))
    return rm, rs, part


def aggregate(unit_len: int, group: int = 1, signal: str = "mass", *,
              q: Optional[torch.Tensor] = None, k: Optional[torch.Tensor] = None,
              v: Optional[torch.Tensor] = None, row_max=None, row_sum=None, part=None,
              scale: Optional[float] = None, cache_shape=None,
              out: Optional[torch.Tensor] = None, accumulate: bool = False) -> torch.Tensor:
    """kvsel_aggregate -> unit_score [B/group][M].

    Chunk path: ``part`` (+ optional row stats), with ``cache_shape`` = k's
    shape or ``k`` given.  Token path: ``q``, ``k`` (``v`` for vnorm) and row stats.
    ``out``: write into this fp32 [B/group][M] tensor; with ``accumulate`` the
    result is added to what it holds."""
    lib = load()
    ref = k if k is not None else None
    if ref is not None:
        kc = cache_desc(ref)
        B, N, H, D = ref.shape
        dev = ref.device
    else:
        B, N, H, D = cache_shape
        dtype = BF16 if q is None or q.dtype == torch.bfloat16 else FP32
        kc = Cache(B, N, H, D, N * H * D, H * D, dtype)
        dev = part.device
    if part is not None:
        _, Hq, T = part.shape[:3]
    else:
        _, T, Hq, _ = q.shape
    scale = 1.0 / D ** 0.5 if scale is None else scale
    if out is None:
        if accumulate:
            raise KvselError(-1, "accumulate needs out")
        out = _empty((B // group, N // unit_len), dev)
    elif (tuple(out.shape) != (B // group, N // unit_len) or out.dtype != torch.float32
          or not out.is_contiguous()):
        raise KvselError(-2, "out must be contiguous fp32 [B/group][M]")
    chunk = signal == "mass" and part is not None
    need = lib.kvsel_aggregate_workspace(B, N, Hq, T, unit_len, int(chunk), int(row_max is not None))
    ws = _workspace(need, dev)
    _check(lib.kvsel_aggregate(_ptr(q), T, Hq, _ptr(k), _ptr(v), kc, scale, _ptr(row_max),
                               _ptr(row_sum), _ptr(part), SIGNAL[signal], unit_len, group,
                               _ptr(out), int(accumulate), _ptr(ws), need, _stream(dev)))
    return out


def topk(scores: torch.Tensor, k: int, values: bool = False):
    """kvsel_topk -> idx int32 [G][k] ascending (and the kept scores if asked)."""
    lib = load()
    G, M = scores.shape
    idx = torch.empty((G, k), dtype=torch.int32, device=scores.device)
    val = _empty((G, k), scores.device) if values else None
    _check(lib.kvsel_topk(_ptr(scores), G, M, k, _ptr(idx), _ptr(val), _stream(scores.device)))
    return (idx, val) if values else idx


def take(src: torch.Tensor, idx: torch.Tensor) -> torch.Tensor:
    """kvsel_take -> out[g][j] = src[g][idx[g][j]] (int32; -1 where idx is out of range)."""
    lib = load()
    G, m = src.shape
    kk = idx.shape[1]
    for t in (src, idx):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise KvselError(-2, "take works on contiguous int32 tensors")
    out = torch.empty((G, kk), dtype=torch.int32, device=src.device)
    _check(lib.kvsel_take(_ptr(src), G, m, _ptr(idx), kk, _ptr(out), _stream(src.device)))
    return out


def order(scores: torch.Tensor, idx: torch.Tensor, descending: bool = True,
          values: bool = False):
    """kvsel_order -> idx listed by score (most relevant first, or last with
    ``descending=False``), and the listed scores if asked."""
    lib = load()
    G, M = scores.shape
    kk = idx.shape[1]
    if idx.dtype != torch.int32 or not idx.is_contiguous() or idx.shape[0] != G:
        raise KvselError(-2, "idx must be contiguous int32 [G][k]")
    out = torch.empty((G, kk), dtype=torch.int32, device=scores.device)
    val = _empty((G, kk), scores.device) if values else None
    _check(lib.kvsel_order(_ptr(scores), G, M, _ptr(idx), kk, int(descending), _ptr(out),
                           _ptr(val), _stream(scores.device)))
    return (out, val) if values else out


def index_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, pos: torch.Tensor,
               scale: Optional[float] = None, want_lse: bool = True):
    """kvsel_index_attn -> (o fp32 [B][S][Hq][D], lse [B][Hq][S] or None): the
    selected tokens' queries ``q`` [B][S][Hq][D] attend to keys 0 .. pos[b][j]."""
    lib = load()
    B, S, Hq, D = q.shape
    if pos.dtype != torch.int32 or tuple(pos.shape) != (B, S) or not pos.is_contiguous():
        raise KvselError(-2, "pos must be contiguous int32 [B][S]")
    if k.shape != v.shape or k.stride() != v.stride():
        raise KvselError(-2, "k and v must share shape and strides")
    scale = 1.0 / D ** 0.5 if scale is None else scale
    out = _empty((B, S, Hq, D), q.device)
    lse = _empty((B, Hq, S), q.device) if want_lse else None
    _check(lib.kvsel_index_attn(_ptr(q), S, Hq, scale, _ptr(k), _ptr(v), cache_desc(k), _ptr(pos),
                                _ptr(out), _ptr(lse), _stream(q.device)))
    return out, lse


def unit_fractions(sel: torch.Tensor, unit_len: int, n_units: int) -> torch.Tensor:
    """kvsel_unit_fractions -> r fp32 [G][n_units]: the share of each unit's
    rows in the ascending index lists ``sel`` (int32 [G][k])."""
    lib = load()
    if sel.dtype != torch.int32 or sel.dim() != 2 or not sel.is_contiguous():
        raise KvselError(-2, "sel must be contiguous int32 [G][k]")
    G, kk = sel.shape
    r = _empty((G, n_units), sel.device)
    _check(lib.kvsel_unit_fractions(_ptr(sel), G, kk, unit_len, n_units, _ptr(r),
                                    _stream(sel.device)))
    return r


def slot_starts(order: torch.Tensor, unit_len: int, rep: int = 1, base: int = 0) -> torch.Tensor:
    """kvsel_slot_starts -> delta int64 [G*rep][M]: each unit's start once the
    units are concatenated in ``order`` (int32 [G][M], a permutation per row)."""
    lib = load()
    if order.dtype != torch.int32 or order.dim() != 2 or not order.is_contiguous():
        raise KvselError(-2, "order must be contiguous int32 [G][M]")
    G, M = order.shape
    delta = torch.empty((G * rep, M), dtype=torch.int64, device=order.device)
    _check(lib.kvsel_slot_starts(_ptr(order), G, M, unit_len, base, rep, _ptr(delta),
                                 _stream(order.device)))
    return delta


def gather(k: torch.Tensor, v: Optional[torch.Tensor], idx: torch.Tensor, unit_len: int,
           idx_group: int = 1, src_start: Optional[torch.Tensor] = None, align_base: int = -1,
           rope_base: float = 10000.0, style: str = "half",
           proxy_k: Optional[torch.Tensor] = None, proxy_v: Optional[torch.Tensor] = None):
    """kvsel_gather -> (k_dst, v_dst): compact, or nested with a proxy cache.
    ``k`` / ``v`` may be pinned host tensors (a host-resident cache); the
    outputs are on the device of ``idx``."""
    lib = load()
    B, N, H, D = k.shape
    kk = idx.shape[1]
    dev = idx.device
    rows = kk * unit_len + (proxy_k.shape[1] if proxy_k is not None else 0)
    kd = torch.empty((B, rows, H, D), dtype=k.dtype, device=dev)
    vd = torch.empty_like(kd) if v is not None else None
    pdesc = ctypes.pointer(cache_desc(proxy_k)) if proxy_k is not None else None
    _check(lib.kvsel_gather(_ptr(k), _ptr(v), cache_desc(k), unit_len, _ptr(idx), kk, idx_group,
                            _ptr(src_start), align_base, rope_base, ROPE[style], _ptr(proxy_k),
                            _ptr(proxy_v), pdesc, _ptr(kd), _ptr(vd), _stream(dev)))
    return kd, vd


def decode_attn(q: torch.Tensor, segments: Sequence[Tuple[torch.Tensor, torch.Tensor]],
                scale: Optional[float] = None, want_lse: bool = True):
    """kvsel_decode_attn -> (o fp32 [B][T][Hq][D], lse [B][Hq][T] or None)."""
    lib = load()
    B, T, Hq, D = q.shape
    scale = 1.0 / D ** 0.5 if scale is None else scale
    segs = (Segment * len(segments))(*[Segment(kk.data_ptr(), vv.data_ptr(), cache_desc(kk))
                                       for kk, vv in segments])
    need = lib.kvsel_decode_workspace(T, Hq, segs, len(segments))
    ws = _workspace(need, q.device)
    out = _empty((B, T, Hq, D), q.device)
    lse = _empty((B, Hq, T), q.device) if want_lse else None
    _check(lib.kvsel_decode_attn(_ptr(q), T, Hq, scale, segs, len(segments), _ptr(out), _ptr(lse),
                                 _ptr(ws), need, _stream(q.device)))
    return out, lse


def gather_decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, idx: torch.Tensor,
                  unit_len: int, idx_group: int = 1,
                  extra: Sequence[Tuple[torch.Tensor, torch.Tensor]] = (),
                  scale: Optional[float] = None, want_lse: bool = True):
    """kvsel_gather_decode -> (k_dst, v_dst, o, lse): the compact cache of the
    kept units and one attention pass over ``extra`` segments plus that cache."""
    lib = load()
    B, T, Hq, D = q.shape
    _, N, H, _ = k.shape
    kk = idx.shape[1]
    scale = 1.0 / D ** 0.5 if scale is None else scale
    kd = torch.empty((B, kk * unit_len, H, D), dtype=k.dtype, device=q.device)
    vd = torch.empty_like(kd)
    n_extra = len(extra)
    segs = (Segment * max(1, n_extra))(*[Segment(a.data_ptr(), b.data_ptr(), cache_desc(a))
                                         for a, b in extra])
    kc = cache_desc(k)
    need = lib.kvsel_gather_decode_workspace(T, Hq, kc, unit_len, kk, segs, n_extra)
    ws = _workspace(need, q.device)
    out = _empty((B, T, Hq, D), q.device)
    lse = _empty((B, Hq, T), q.device) if want_lse else None
    _check(lib.kvsel_gather_decode(_ptr(q), T, Hq, scale, _ptr(k), _ptr(v), kc, unit_len,
                                   _ptr(idx), kk, idx_group, _ptr(kd), _ptr(vd), segs, n_extra,
                                   _ptr(out), _ptr(lse), _ptr(ws), need, _stream(q.device)))
    return kd, vd, out, lse
