"""Python binding of libkvsel (ctypes).  Argument marshalling only.

Each function mirrors one C entry point of ``include/kvsel.h``: it takes torch
tensors that live on the GPU, checks that they have the shapes, dtypes,
layouts and devices the entry point reads, allocates the outputs and
workspace it is not given (torch's caching allocator), passes raw device
pointers and the current HIP stream, and raises :class:`KvselError` on a
negative status.  A tensor that does not fit is refused here, before any
pointer reaches the library.  All computation happens in the library's
kernels; there is no fallback.

Every output (and the workspace, a uint8 tensor) may be passed in instead of
allocated, so that a loop of calls allocates nothing per step and can be
captured as a HIP graph.
"""

from __future__ import annotations

import ctypes
from typing import Optional, Sequence, Tuple

import torch

from .abi import (BF16, FP32, LIB_PATH, ROPE, SIGNAL, Cache, Segment, load,  # noqa: F401
                  ERR_DTYPE, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_WORKSPACE)


class KvselError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"kvsel status {status}: {msg}")
        self.status = status


def _check(rc: int) -> None:
    if rc != 0:
        lib = load()
        raise KvselError(rc, f"{lib.kvsel_status_str(rc).decode()}: {lib.kvsel_last_error().decode()}")


_recorder: Optional[list] = None


def _invoke(fn, *args) -> None:
    """Call a library entry point with its marshalled arguments (recorded
    first when a :class:`Recording` is active) and check the status."""
    if _recorder is not None:
        _recorder.append((fn, args))
    _check(fn(*args))


class Recording:
    """Collects the (entry point, arguments) of every library call made inside
    the ``with`` block, so that a caller whose arguments stay the same can
    replay them with :func:`replay`, skipping the checks that already passed."""

    def __enter__(self) -> list:
        global _recorder
        self._prev, self.calls = _recorder, []
        _recorder = self.calls
        return self.calls

    def __exit__(self, *exc) -> None:
        global _recorder
        _recorder = self._prev


def replay(calls: list) -> None:
    """Make the recorded library calls again, with the same arguments."""
    for fn, args in calls:
        _check(fn(*args))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return FP32
    raise KvselError(ERR_DTYPE, f"unsupported dtype {t.dtype}")


def cache_desc(t: torch.Tensor) -> Cache:
    """Descriptor of a [B][N][H][D] tensor whose [H][D] block is contiguous."""
    if t.dim() != 4:
        raise KvselError(ERR_SHAPE, f"cache must be [B][N][H][D], got {tuple(t.shape)}")
    B, N, H, D = t.shape
    if t.stride(3) != 1 or t.stride(2) != D:
        raise KvselError(ERR_UNSUPPORTED, "cache rows must hold contiguous [H][D]")
    return Cache(B, N, H, D, t.stride(0), t.stride(1), dtype_code(t))


# ---------------------------------------------------------------------------
# argument checks (all raise KvselError before anything is launched)
# ---------------------------------------------------------------------------

def _gpu(**tensors) -> None:
    """Checked after every shape and dtype check: the named tensors are GPU
    memory (a CPU tensor never reaches the library)."""
    for name, t in tensors.items():
        if t is not None and t.device.type != "cuda":
            raise KvselError(ERR_UNSUPPORTED, f"{name} must be GPU memory, got {t.device}")


def _same_device(t: torch.Tensor, dev: torch.device, name: str) -> None:
    if t.device != dev:
        raise KvselError(ERR_UNSUPPORTED, f"{name} is on {t.device}, expected {dev}")


def _source_device(t: torch.Tensor, dev: torch.device, name: str) -> None:
    """Gather sources may also be pinned host memory (a host-resident cache)."""
    if t.device != dev and not (t.device.type == "cpu" and t.is_pinned()):
        raise KvselError(ERR_UNSUPPORTED,
                         f"{name} must be on {dev} or in pinned host memory, got {t.device}")


def _check_query(q: torch.Tensor, ref: torch.Tensor, name: str = "q",
                 same_device: bool = True) -> Tuple[int, int]:
    """q is a contiguous [B][T][Hq][D] block in ref's dtype (and on its device
    unless the cache may be host memory), for a cache ref [B][N][H][D] (Hq a
    multiple of H); returns (T, Hq)."""
    if q.dim() != 4:
        raise KvselError(ERR_SHAPE, f"{name} must be [B][T][Hq][D], got {tuple(q.shape)}")
    B, _, H, D = ref.shape
    if q.shape[0] != B or q.shape[3] != D or q.shape[1] < 1 or q.shape[2] < 1 \
            or q.shape[2] % H != 0:
        raise KvselError(ERR_SHAPE, f"{name} {tuple(q.shape)} does not fit cache {tuple(ref.shape)} "
                                    "(same B and D, Hq a multiple of H)")
    if q.dtype != ref.dtype:
        raise KvselError(ERR_DTYPE, f"{name} is {q.dtype}, the cache {ref.dtype}")
    if same_device and q.device != ref.device:
        raise KvselError(ERR_UNSUPPORTED, f"{name} is on {q.device}, the cache on {ref.device}")
    if not q.is_contiguous():
        raise KvselError(ERR_UNSUPPORTED, f"{name} must be contiguous")
    return q.shape[1], q.shape[2]


def _check_like(t: torch.Tensor, ref: torch.Tensor, name: str, ref_name: str = "k") -> None:
    """t has ref's shape, strides, dtype and device (a value cache beside its keys)."""
    if tuple(t.shape) != tuple(ref.shape) or t.stride() != ref.stride():
        raise KvselError(ERR_SHAPE, f"{name} must match {ref_name} in shape and strides")
    if t.dtype != ref.dtype:
        raise KvselError(ERR_DTYPE, f"{name} is {t.dtype}, {ref_name} is {ref.dtype}")
    if t.device != ref.device:
        raise KvselError(ERR_UNSUPPORTED, f"{name} is on {t.device}, {ref_name} on {ref.device}")


def _check_tensor(t: torch.Tensor, shape, dtype, dev: torch.device, name: str) -> None:
    """A contiguous tensor of exactly this shape and dtype on dev."""
    if t.dtype != dtype:
        raise KvselError(ERR_DTYPE, f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise KvselError(ERR_SHAPE, f"{name} must be {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise KvselError(ERR_UNSUPPORTED, f"{name} must be contiguous")
    _same_device(t, dev, name)


def _check_delta(delta: torch.Tensor, B: int, M: int, dev: torch.device) -> int:
    """int64 [M] (shared) or [B][M] (per instance); returns the per-instance flag."""
    if delta.dim() == 1:
        _check_tensor(delta, (M,), torch.int64, dev, "delta")
        return 0
    _check_tensor(delta, (B, M), torch.int64, dev, "delta")
    return 1


def _check_idx(idx: torch.Tensor, B: int, idx_group: int, dev: torch.device) -> int:
    """int32 [B/idx_group][k]; returns k."""
    if idx_group < 1 or B % idx_group != 0:
        raise KvselError(ERR_SHAPE, f"idx_group {idx_group} must divide B={B}")
    if idx.dim() != 2:
        raise KvselError(ERR_SHAPE, f"idx must be [B/idx_group][k], got {tuple(idx.shape)}")
    _check_tensor(idx, (B // idx_group, idx.shape[1]), torch.int32, dev, "idx")
    return idx.shape[1]


def _out(t: Optional[torch.Tensor], shape, dtype, dev, name: str) -> torch.Tensor:
    """The caller's output tensor, checked, or a new one."""
    if t is None:
        return torch.empty(shape, dtype=dtype, device=dev)
    _check_tensor(t, shape, dtype, dev, name)
    return t


class Workspace:
    """A workspace kept across calls: allocated by the first call that needs
    it and grown only when a call needs more, so that a loop of identical
    calls allocates once (and a HIP graph captured after the first call
    allocates nothing)."""

    def __init__(self):
        self.tensor: Optional[torch.Tensor] = None

    def get(self, nbytes: int, dev) -> Optional[torch.Tensor]:
        if nbytes == 0:
            return None
        t = self.tensor
        if t is None or t.numel() < nbytes or t.device != dev:
            t = torch.empty((nbytes + 255) // 256 * 256, dtype=torch.uint8, device=dev)
            self.tensor = t
        return t


def _workspace(nbytes: int, dev, ws=None) -> Optional[torch.Tensor]:
    """The caller's uint8 workspace (at least nbytes; a tensor or a
    :class:`Workspace`), or a new one."""
    if isinstance(ws, Workspace):
        return ws.get(nbytes, dev)
    if ws is not None:
        if ws.dtype != torch.uint8 or not ws.is_contiguous() or ws.numel() < nbytes:
            raise KvselError(ERR_WORKSPACE, f"workspace must be contiguous uint8 of at least "
                                            f"{nbytes} bytes")
        _same_device(ws, dev, "workspace")
        return ws
    return torch.empty(max(1, (nbytes + 255) // 256 * 256), dtype=torch.uint8, device=dev) if nbytes else None


def _nbytes(ws: Optional[torch.Tensor]) -> int:
    return 0 if ws is None else ws.numel()


def _scale(scale: Optional[float], D: int) -> float:
    return 1.0 / D ** 0.5 if scale is None else scale


# ---------------------------------------------------------------------------
# the six calls
# ---------------------------------------------------------------------------

def reposition(k: torch.Tensor, delta: torch.Tensor, unit_len: int,
               out: Optional[torch.Tensor] = None, rope_base: float = 10000.0,
               style: str = "half") -> torch.Tensor:
    """kvsel_reposition: rotate every row of unit u by delta[u] positions.
    ``delta``: int64 [M] or [B][M] on the device.  ``out`` may be ``k`` (in place)."""
    lib = load()
    kc = cache_desc(k)
    dev = k.device
    if unit_len < 1 or k.shape[1] % unit_len:
        raise KvselError(ERR_SHAPE, f"unit_len {unit_len} must divide N={k.shape[1]}")
    per = _check_delta(delta, k.shape[0], k.shape[1] // unit_len, dev)
    if out is None:
        out = torch.empty_like(k)
    else:
        _check_like(out, k, "out")
    _gpu(k=k, delta=delta, out=out)
    _invoke(lib.kvsel_reposition, _ptr(k), _ptr(out), kc, unit_len, _ptr(delta), per,
                                rope_base, ROPE[style], _stream(dev))
    return out


def _stat_outs(B, Hq, T, M, dev, row_stats, partials, rm, rs, part):
    rm = _out(rm, (B, Hq, T), torch.float32, dev, "row_max") if row_stats else None
    rs = _out(rs, (B, Hq, T), torch.float32, dev, "row_sum") if row_stats else None
    part = _out(part, (B, Hq, T, M, 2), torch.float32, dev, "part") if partials else None
    return rm, rs, part


def score(q: torch.Tensor, k: torch.Tensor, unit_len: int, scale: Optional[float] = None,
          row_stats: bool = True, partials: bool = True, *, rm_out=None, rs_out=None,
          part_out=None, ws=None):
    """kvsel_score -> (row_max, row_sum, part); entries not requested are None."""
    lib = load()
    kc = cache_desc(k)
    dev = k.device
    T, Hq = _check_query(q, k)
    B, N, _, D = k.shape
    if unit_len < 1 or N % unit_len:
        raise KvselError(ERR_SHAPE, f"unit_len {unit_len} must divide N={N}")
    rm, rs, part = _stat_outs(B, Hq, T, N // unit_len, dev, row_stats, partials, rm_out, rs_out,
                              part_out)
    need = lib.kvsel_score_workspace(B, N, Hq, T, unit_len, int(row_stats), int(partials))
    ws = _workspace(need, dev, ws)
    _gpu(q=q, k=k)
    _invoke(lib.kvsel_score, _ptr(q), T, Hq, _ptr(k), kc, _scale(scale, D), unit_len, _ptr(rm),
                           _ptr(rs), _ptr(part), _ptr(ws), _nbytes(ws), _stream(dev))
    return rm, rs, part


def score_reposition(q: torch.Tensor, k: torch.Tensor, delta: torch.Tensor, rot_unit_len: int,
                     unit_len: int, k_out: Optional[torch.Tensor] = None,
                     scale: Optional[float] = None, row_stats: bool = True,
                     partials: bool = True, rope_base: float = 10000.0, style: str = "half",
                     *, rm_out=None, rs_out=None, part_out=None, ws=None):
    """kvsel_score_reposition -> (row_max, row_sum, part) of the keys rotated by
    delta[u] per unit of ``rot_unit_len`` rows; ``k_out`` (same shape and strides
    as ``k``) receives the re-positioned keys when given."""
    lib = load()
    kc = cache_desc(k)
    dev = k.device
    T, Hq = _check_query(q, k)
    B, N, _, D = k.shape
    if unit_len < 1 or N % unit_len or rot_unit_len < 1 or N % rot_unit_len:
        raise KvselError(ERR_SHAPE, f"unit_len {unit_len} and rot_unit_len {rot_unit_len} "
                                    f"must divide N={N}")
    per = _check_delta(delta, B, N // rot_unit_len, dev)
    if k_out is not None:
        _check_like(k_out, k, "k_out")
    rm, rs, part = _stat_outs(B, Hq, T, N // unit_len, dev, row_stats, partials, rm_out, rs_out,
                              part_out)
    need = lib.kvsel_score_reposition_workspace(T, Hq, kc, unit_len, rot_unit_len,
                                                int(row_stats), int(partials),
                                                int(k_out is not None))
    ws = _workspace(need, dev, ws)
    _gpu(q=q, k=k)
    _invoke(lib.kvsel_score_reposition, _ptr(q), T, Hq, _ptr(k), _ptr(k_out), kc, _scale(scale, D),
                                      unit_len, rot_unit_len, _ptr(delta), per, rope_base,
                                      ROPE[style], _ptr(rm), _ptr(rs), _ptr(part), _ptr(ws),
                                      _nbytes(ws), _stream(dev))
    return rm, rs, part


def score_units(q: torch.Tensor, k: torch.Tensor, units: torch.Tensor, unit_len: int,
                delta: Optional[torch.Tensor] = None, scale: Optional[float] = None,
                row_stats: bool = True, partials: bool = True, rope_base: float = 10000.0,
                style: str = "half", *, rm_out=None, rs_out=None, part_out=None, ws=None):
    """kvsel_score_units -> (row_max, row_sum, part) of each instance's query
    block against the listed units of its cache (``units`` int32 [B][n]), unit
    j re-positioned by ``delta[j]`` (int64 [n] or [B][n]) when given.  ``k``
    may be a strided view, e.g. one layer of a [R][L][N][H][D] store."""
    lib = load()
    kc = cache_desc(k)
    dev = k.device
    T, Hq = _check_query(q, k)
    B, _, _, D = k.shape
    if units.dim() != 2:
        raise KvselError(ERR_SHAPE, "units must be contiguous int32 [B][n_units]")
    n = units.shape[1]
    _check_tensor(units, (B, n), torch.int32, dev, "units")
    per = 0 if delta is None else _check_delta(delta, B, n, dev)
    rm, rs, part = _stat_outs(B, Hq, T, n, dev, row_stats, partials, rm_out, rs_out, part_out)
    need = lib.kvsel_score_units_workspace(T, Hq, kc, unit_len, n, int(row_stats), int(partials))
    ws = _workspace(need, dev, ws)
    _gpu(q=q, k=k)
    _invoke(lib.kvsel_score_units, _ptr(q), T, Hq, _ptr(k), kc, _scale(scale, D), unit_len,
                                 _ptr(units), n, _ptr(delta), per, rope_base, ROPE[style],
                                 _ptr(rm), _ptr(rs), _ptr(part), _ptr(ws), _nbytes(ws),
                                 _stream(dev))
    return rm, rs, part


def aggregate(unit_len: int, group: int = 1, signal: str = "mass", *,
              q: Optional[torch.Tensor] = None, k: Optional[torch.Tensor] = None,
              v: Optional[torch.Tensor] = None, row_max=None, row_sum=None, part=None,
              scale: Optional[float] = None, cache_shape=None,
              out: Optional[torch.Tensor] = None, accumulate: bool = False,
              ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """kvsel_aggregate -> unit_score [B/group][M].

    Chunk path: ``part`` (+ optional row stats), with ``cache_shape`` = k's
    shape or ``k`` given.  Token path: ``q``, ``k`` (``v`` for vnorm) and row stats.
    ``out``: write into this fp32 [B/group][M] tensor; with ``accumulate`` the
    result is added to what it holds."""
    lib = load()
    chunk = signal == "mass" and part is not None
    if k is not None:
        kc = cache_desc(k)
        B, N, H, D = k.shape
        dev = k.device
    else:
        if not chunk or cache_shape is None:
            raise KvselError(ERR_NULL, "the token path needs k (and q, row statistics)")
        B, N, H, D = cache_shape
        dtype = BF16 if q is None or q.dtype == torch.bfloat16 else FP32
        kc = Cache(B, N, H, D, N * H * D, H * D, dtype)
        dev = part.device
    if unit_len < 1 or N % unit_len:
        raise KvselError(ERR_SHAPE, f"unit_len {unit_len} must divide N={N}")
    if group < 1 or B % group:
        raise KvselError(ERR_SHAPE, f"group {group} must divide B={B}")
    M = N // unit_len
    if chunk:
        if part.dim() != 5:
            raise KvselError(ERR_SHAPE, "part must be [B][Hq][T][M][2]")
        Hq, T = part.shape[1], part.shape[2]
        _check_tensor(part, (B, Hq, T, M, 2), torch.float32, dev, "part")
    else:
        if q is None or row_max is None or row_sum is None:
            raise KvselError(ERR_NULL, "the token path needs q, k and the row statistics")
        T, Hq = _check_query(q, k)
        if signal == "vnorm":
            if v is None:
                raise KvselError(ERR_NULL, "the vnorm signal needs v")
            _check_like(v, k, "v")
    if (row_max is None) != (row_sum is None):
        raise KvselError(ERR_NULL, "row_max and row_sum must both be given or both omitted")
    if row_max is not None:
        _check_tensor(row_max, (B, Hq, T), torch.float32, dev, "row_max")
        _check_tensor(row_sum, (B, Hq, T), torch.float32, dev, "row_sum")
    if out is None and accumulate:
        raise KvselError(ERR_NULL, "accumulate needs out")
    out = _out(out, (B // group, M), torch.float32, dev, "out")
    need = lib.kvsel_aggregate_workspace(B, N, Hq, T, unit_len, int(chunk), int(row_max is not None))
    ws = _workspace(need, dev, ws)
    _gpu(out=out, part=part, k=k)
    _invoke(lib.kvsel_aggregate, _ptr(q), T, Hq, _ptr(k), _ptr(v), kc, _scale(scale, D),
                               _ptr(row_max), _ptr(row_sum), _ptr(part), SIGNAL[signal], unit_len,
                               group, _ptr(out), int(accumulate), _ptr(ws), _nbytes(ws),
                               _stream(dev))
    return out


def _check_scores(scores: torch.Tensor, name: str = "scores") -> Tuple[int, int]:
    dev = scores.device
    if scores.dim() != 2:
        raise KvselError(ERR_SHAPE, f"{name} must be fp32 [G][M], got {tuple(scores.shape)}")
    _check_tensor(scores, scores.shape, torch.float32, dev, name)
    return scores.shape


def topk(scores: torch.Tensor, k: int, values: bool = False, *, idx_out=None, val_out=None):
    """kvsel_topk -> idx int32 [G][k] ascending (and the kept scores if asked)."""
    lib = load()
    G, M = _check_scores(scores)
    dev = scores.device
    idx = _out(idx_out, (G, k), torch.int32, dev, "idx")
    val = _out(val_out, (G, k), torch.float32, dev, "val") if values else None
    _gpu(scores=scores)
    _invoke(lib.kvsel_topk, _ptr(scores), G, M, k, _ptr(idx), _ptr(val), _stream(dev))
    return (idx, val) if values else idx


def take(src: torch.Tensor, idx: torch.Tensor) -> torch.Tensor:
    """kvsel_take -> out[g][j] = src[g][idx[g][j]] (int32; -1 where idx is out of range)."""
    lib = load()
    dev = src.device
    if src.dim() != 2 or idx.dim() != 2 or idx.shape[0] != src.shape[0]:
        raise KvselError(ERR_SHAPE, "take works on int32 [G][m] and [G][k]")
    _check_tensor(src, src.shape, torch.int32, dev, "src")
    _check_tensor(idx, idx.shape, torch.int32, dev, "idx")
    G, m = src.shape
    kk = idx.shape[1]
    out = torch.empty((G, kk), dtype=torch.int32, device=dev)
    _gpu(src=src)
    _invoke(lib.kvsel_take, _ptr(src), G, m, _ptr(idx), kk, _ptr(out), _stream(dev))
    return out


def order(scores: torch.Tensor, idx: torch.Tensor, descending: bool = True,
          values: bool = False):
    """kvsel_order -> idx listed by score (most relevant first, or last with
    ``descending=False``), and the listed scores if asked."""
    lib = load()
    G, M = _check_scores(scores)
    dev = scores.device
    if idx.dim() != 2:
        raise KvselError(ERR_SHAPE, "idx must be contiguous int32 [G][k]")
    kk = idx.shape[1]
    _check_tensor(idx, (G, kk), torch.int32, dev, "idx")
    out = torch.empty((G, kk), dtype=torch.int32, device=dev)
    val = torch.empty((G, kk), dtype=torch.float32, device=dev) if values else None
    _gpu(scores=scores)
    _invoke(lib.kvsel_order, _ptr(scores), G, M, _ptr(idx), kk, int(descending), _ptr(out),
                           _ptr(val), _stream(dev))
    return (out, val) if values else out


def index_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, pos: torch.Tensor,
               scale: Optional[float] = None, want_lse: bool = True):
    """kvsel_index_attn -> (o fp32 [B][S][Hq][D], lse [B][Hq][S] or None): the
    selected tokens' queries ``q`` [B][S][Hq][D] attend to keys 0 .. pos[b][j]."""
    lib = load()
    kc = cache_desc(k)
    dev = k.device
    _check_like(v, k, "v")
    S, Hq = _check_query(q, k)
    B, _, _, D = k.shape
    _check_tensor(pos, (B, S), torch.int32, dev, "pos")
    out = torch.empty((B, S, Hq, D), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=dev) if want_lse else None
    _gpu(q=q, k=k)
    _invoke(lib.kvsel_index_attn, _ptr(q), S, Hq, _scale(scale, D), _ptr(k), _ptr(v), kc, _ptr(pos),
                                _ptr(out), _ptr(lse), _stream(dev))
    return out, lse


def unit_fractions(sel: torch.Tensor, unit_len: int, n_units: int) -> torch.Tensor:
    """kvsel_unit_fractions -> r fp32 [G][n_units]: the share of each unit's
    rows in the ascending index lists ``sel`` (int32 [G][k])."""
    lib = load()
    dev = sel.device
    if sel.dim() != 2:
        raise KvselError(ERR_SHAPE, "sel must be contiguous int32 [G][k]")
    _check_tensor(sel, sel.shape, torch.int32, dev, "sel")
    G, kk = sel.shape
    r = torch.empty((G, n_units), dtype=torch.float32, device=dev)
    _gpu(sel=sel)
    _invoke(lib.kvsel_unit_fractions, _ptr(sel), G, kk, unit_len, n_units, _ptr(r), _stream(dev))
    return r


def slot_starts(order: torch.Tensor, unit_len: int, rep: int = 1, base: int = 0) -> torch.Tensor:
    """kvsel_slot_starts -> delta int64 [G*rep][M]: each unit's start once the
    units are concatenated in ``order`` (int32 [G][M], a permutation per row)."""
    lib = load()
    dev = order.device
    if order.dim() != 2:
        raise KvselError(ERR_SHAPE, "order must be contiguous int32 [G][M]")
    _check_tensor(order, order.shape, torch.int32, dev, "order")
    G, M = order.shape
    delta = torch.empty((G * rep, M), dtype=torch.int64, device=dev)
    _gpu(order=order)
    _invoke(lib.kvsel_slot_starts, _ptr(order), G, M, unit_len, base, rep, _ptr(delta),
                                 _stream(dev))
    return delta


def gather(k: torch.Tensor, v: Optional[torch.Tensor], idx: torch.Tensor, unit_len: int,
           idx_group: int = 1, src_start: Optional[torch.Tensor] = None, align_base: int = -1,
           rope_base: float = 10000.0, style: str = "half",
           proxy_k: Optional[torch.Tensor] = None, proxy_v: Optional[torch.Tensor] = None,
           *, k_out=None, v_out=None):
    """kvsel_gather -> (k_dst, v_dst): compact, or nested with a proxy cache.
    ``k`` / ``v`` may be pinned host tensors (a host-resident cache); the
    outputs are on the device of ``idx``."""
    lib = load()
    kc = cache_desc(k)
    dev = idx.device
    _source_device(k, dev, "k")
    if v is not None:
        _check_like(v, k, "v")
    B, N, H, D = k.shape
    if unit_len < 1 or N % unit_len:
        raise KvselError(ERR_SHAPE, f"unit_len {unit_len} must divide N={N}")
    kk = _check_idx(idx, B, idx_group, dev)
    if src_start is not None:
        _check_tensor(src_start, (N // unit_len,), torch.int64, dev, "src_start")
    pdesc = None
    if proxy_k is not None:
        pdesc = ctypes.pointer(cache_desc(proxy_k))
        _same_device(proxy_k, dev, "proxy_k")
        if (proxy_v is None) != (v is None):
            raise KvselError(ERR_NULL, "proxy_v must be given exactly when v is")
        if proxy_v is not None:
            _check_like(proxy_v, proxy_k, "proxy_v", "proxy_k")
    rows = kk * unit_len + (proxy_k.shape[1] if proxy_k is not None else 0)
    kd = _out(k_out, (B, rows, H, D), k.dtype, dev, "k_out")
    vd = _out(v_out, (B, rows, H, D), k.dtype, dev, "v_out") if v is not None else None
    _gpu(idx=idx)
    _invoke(lib.kvsel_gather, _ptr(k), _ptr(v), kc, unit_len, _ptr(idx), kk, idx_group,
                            _ptr(src_start), align_base, rope_base, ROPE[style], _ptr(proxy_k),
                            _ptr(proxy_v), pdesc, _ptr(kd), _ptr(vd), _stream(dev))
    return kd, vd


def _segments(q: torch.Tensor, pairs: Sequence[Tuple[torch.Tensor, torch.Tensor]], name: str):
    """ctypes segment array of (k, v) pairs that the query block q attends."""
    for i, (kk, vv) in enumerate(pairs):
        cache_desc(kk)
        k0 = pairs[0][0]
        if (kk.shape[0], kk.shape[2], kk.shape[3], kk.dtype) != \
                (k0.shape[0], k0.shape[2], k0.shape[3], k0.dtype):
            raise KvselError(ERR_SHAPE, f"{name}: segments must share B, H, D and dtype")
        _check_like(vv, kk, f"{name}[{i}] v", f"{name}[{i}] k")
        _same_device(kk, q.device, f"{name}[{i}] k")
        _check_query(q, kk)
    return (Segment * max(1, len(pairs)))(*[Segment(kk.data_ptr(), vv.data_ptr(), cache_desc(kk))
                                            for kk, vv in pairs])


def decode_attn(q: torch.Tensor, segments: Sequence[Tuple[torch.Tensor, torch.Tensor]],
                scale: Optional[float] = None, want_lse: bool = True, *, out=None, lse_out=None,
                ws=None):
    """kvsel_decode_attn -> (o fp32 [B][T][Hq][D], lse [B][Hq][T] or None)."""
    lib = load()
    if not segments:
        raise KvselError(ERR_SHAPE, "decode_attn needs at least one segment")
    segs = _segments(q, segments, "segments")
    B, T, Hq, D = q.shape
    dev = q.device
    need = lib.kvsel_decode_workspace(T, Hq, segs, len(segments))
    ws = _workspace(need, dev, ws)
    o = _out(out, (B, T, Hq, D), torch.float32, dev, "out")
    lse = _out(lse_out, (B, Hq, T), torch.float32, dev, "lse") if want_lse else None
    _gpu(q=q)
    _invoke(lib.kvsel_decode_attn, _ptr(q), T, Hq, _scale(scale, D), segs, len(segments), _ptr(o),
                                 _ptr(lse), _ptr(ws), _nbytes(ws), _stream(dev))
    return o, lse


def gather_decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, idx: torch.Tensor,
                  unit_len: int, idx_group: int = 1,
                  extra: Sequence[Tuple[torch.Tensor, torch.Tensor]] = (),
                  scale: Optional[float] = None, want_lse: bool = True, *, k_out=None,
                  v_out=None, out=None, lse_out=None, ws=None):
    """kvsel_gather_decode -> (k_dst, v_dst, o, lse): the compact cache of the
    kept units and one attention pass over ``extra`` segments plus that cache."""
    lib = load()
    kc = cache_desc(k)
    dev = q.device
    _source_device(k, dev, "k")
    _check_like(v, k, "v")
    _check_query(q, k, same_device=False)
    B, T, Hq, D = q.shape
    _, N, H, _ = k.shape
    if unit_len < 1 or N % unit_len:
        raise KvselError(ERR_SHAPE, f"unit_len {unit_len} must divide N={N}")
    kk = _check_idx(idx, B, idx_group, dev)
    n_extra = len(extra)
    segs = _segments(q, extra, "extra")
    kd = _out(k_out, (B, kk * unit_len, H, D), k.dtype, dev, "k_out")
    vd = _out(v_out, (B, kk * unit_len, H, D), k.dtype, dev, "v_out")
    need = lib.kvsel_gather_decode_workspace(T, Hq, kc, unit_len, kk, segs, n_extra)
    ws = _workspace(need, dev, ws)
    o = _out(out, (B, T, Hq, D), torch.float32, dev, "out")
    lse = _out(lse_out, (B, Hq, T), torch.float32, dev, "lse") if want_lse else None
    _gpu(q=q)
    _invoke(lib.kvsel_gather_decode, _ptr(q), T, Hq, _scale(scale, D), _ptr(k), _ptr(v), kc,
                                   unit_len, _ptr(idx), kk, idx_group, _ptr(kd), _ptr(vd), segs,
                                   n_extra, _ptr(o), _ptr(lse), _ptr(ws), _nbytes(ws),
                                   _stream(dev))
    return kd, vd, o, lse


def gather_decode_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, idx: torch.Tensor,
                          unit_len: int, idx_group: int = 1,
                          extra: Sequence[Tuple[torch.Tensor, torch.Tensor]] = (),
                          scale: Optional[float] = None, want_lse: bool = True, *, k_out=None,
                          v_out=None, out=None, lse_out=None):
    """kvsel_gather_decode_noalloc -> (k_dst, v_dst, o, lse): kvsel_gather_decode
    with its scratch in the library's fixed device array (the call allocates
    nothing; pass every output to allocate nothing here either)."""
    lib = load()
    kc = cache_desc(k)
    dev = q.device
    _source_device(k, dev, "k")
    _check_like(v, k, "v")
    _check_query(q, k, same_device=False)
    B, T, Hq, D = q.shape
    _, N, H, _ = k.shape
    if unit_len < 1 or N % unit_len:
        raise KvselError(ERR_SHAPE, f"unit_len {unit_len} must divide N={N}")
    kk = _check_idx(idx, B, idx_group, dev)
    n_extra = len(extra)
    segs = _segments(q, extra, "extra")
    kd = _out(k_out, (B, kk * unit_len, H, D), k.dtype, dev, "k_out")
    vd = _out(v_out, (B, kk * unit_len, H, D), k.dtype, dev, "v_out")
    o = _out(out, (B, T, Hq, D), torch.float32, dev, "out")
    lse = _out(lse_out, (B, Hq, T), torch.float32, dev, "lse") if want_lse else None
    _gpu(q=q)
    _invoke(lib.kvsel_gather_decode_noalloc, _ptr(q), T, Hq, _scale(scale, D), _ptr(k), _ptr(v), kc,
                                           unit_len, _ptr(idx), kk, idx_group, _ptr(kd),
                                           _ptr(vd), segs, n_extra, _ptr(o), _ptr(lse),
                                           _stream(dev))
    return kd, vd, o, lse


def workspace_bytes(call: str, *args) -> int:
    """The library's workspace query of a call (e.g. ``"gather_decode"``), for
    callers that allocate a workspace once and pass it to every step."""
    return int(getattr(load(), f"kvsel_{call}_workspace")(*args))
