"""Plain fp64 CPU oracle of query-guided KV selection.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  It shares no code
with the HIP library.

Sources, cited below by short name plus section / equation:

* [ACRE] "Boosting Long-Context Management via Query-Guided Activation
  Refilling" (arXiv 2412.12486).
* [CacheFocus] "CacheFocus: Dynamic Cache Re-Positioning for Efficient
  Retrieval-Augmented Generation" (arXiv 2502.11101).
* [InfoFlow] "InfoFlow KV: Information-Flow-Aware KV Recomputation for Long
  Context" (arXiv 2603.05353).

Layout conventions (shared with the library only as a written contract):

* cached keys / values ``k, v``: ``[B][N][H][D]`` (instance, cached row, kv head,
  head dim);
* queries ``q``: ``[B][T][Hq][D]``;
* per-row statistics: ``[B][Hq][T]``; a "row" is one (query head, query token);
* grouped-query attention: query head ``h`` reads kv head ``h // (Hq // H)``.

Every function computes in float64 from the (already rounded) inputs it is
given.  Where the pages leave a step open, the reading taken is stated in the
function's docstring.

Parity status: every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_*.py`` (closed forms, invariants, worked examples printed on
the pages, library routines and brute force).  No function is parity unpinned.
"""

from __future__ import annotations

import math
from fractions import Fraction
from typing import Iterable, Sequence

import numpy as np

__all__ = [
    "round_bf16", "round_to", "rope_theta", "rope_pairs", "rope_rotate",
    "reposition", "logits", "attention_weights", "score", "combine_partials",
    "aggregate", "acre_mean_pool", "topk", "gather", "gather_aligned",
    "refill_nested", "decode_attention", "index_causal_attention", "acre_k", "cf_group_size",
    "cf_reuse_count", "cf_doc_starts", "cf_k_prune", "cf_prune_layers",
    "cf_keep_schedule", "cf_progressive_prune", "cf_final_cache", "take", "order",
    "if_chunk_offsets",
    "if_global_positions", "if_budget", "if_chunk_fractions", "if_reorder",
    "if_reordered_offsets", "if_two_stage",
]


# ---------------------------------------------------------------------------
# Rounding to the cache dtype
# ---------------------------------------------------------------------------

_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def round_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bfloat16 keeps 8 significant bits and float32's exponent range.  A value in
    ``[2**(e-1), 2**e)`` is rounded to a multiple of ``2**(e-8)``; below the
    smallest normal ``2**-126`` the spacing stays ``2**-133``.  Rounding is done
    once, directly from float64 (no float32 intermediate).  Returns float64.
    """
    x = np.asarray(x, dtype=np.float64)
    fin = np.isfinite(x)
    xf = np.where(fin, x, 0.0)
    _, e = np.frexp(xf)
    e = np.maximum(e, -125)
    quantum = np.ldexp(1.0, e - 8)
    r = np.rint(xf / quantum) * quantum          # np.rint rounds half to even
    r = np.where(np.abs(r) > _BF16_MAX, np.copysign(np.inf, r), r)
    return np.where(fin, r, x)


def round_to(x, dtype: str) -> np.ndarray:
    """Round to the cache dtype ("bf16" or "fp32"), ties to even; float64 out.
    "fp64" leaves the values as they are."""
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "fp32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    if dtype == "fp64":     # no rounding (exact checks of the arithmetic)
        return np.asarray(x, dtype=np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# ---------------------------------------------------------------------------
# Rotary position embedding and cache re-positioning
# ---------------------------------------------------------------------------

def rope_theta(D: int, base: float = 10000.0) -> np.ndarray:
    """Per-pair angular frequencies ``theta_i = base**(-2i/D)``, i = 0..D/2-1.

    [InfoFlow §3.2] gives the 2x2 rotation by ``theta_i * t`` but leaves theta_i
    undefined; the standard RoPE frequencies with base 10000 are the reading.
    """
    i = np.arange(D // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / D)


def rope_pairs(D: int, style: str):
    """The two halves (first, second) of the 2-D slices that RoPE rotates, as
    slices of the last axis: pair i is (first[i], second[i]).

    "half": pair i is (i, i + D/2); "interleaved": pair i is (2i, 2i + 1).
    """
    if style == "half":
        return slice(0, D // 2), slice(D // 2, D)
    if style == "interleaved":
        return slice(0, D, 2), slice(1, D, 2)
    raise ValueError(f"unknown rope style {style!r}")


def rope_rotate(x, pos, base: float = 10000.0, style: str = "half",
                transpose: bool = False) -> np.ndarray:
    """Apply the RoPE matrix at position ``pos`` to the last axis of ``x``.

    [InfoFlow §3.2]: each 2-D slice (a, b) maps to
    ``[[cos(theta_i t), -sin(theta_i t)], [sin(theta_i t), cos(theta_i t)]] (a, b)``.
    With ``transpose=True`` the transposed matrix is applied, which is the
    inverse rotation ([CacheFocus §2.3]).  ``pos`` broadcasts against
    ``x.shape[:-1]``; angles are formed in float64.
    """
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    theta = rope_theta(D, base)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * theta
    c, s = np.cos(ang), np.sin(ang)
    f, g = rope_pairs(D, style)
    a, b = x[..., f], x[..., g]
    out = np.empty(np.broadcast_shapes(x.shape, ang.shape[:-1] + (D,)), dtype=np.float64)
    if not transpose:
        out[..., f] = c * a - s * b
        out[..., g] = s * a + c * b
    else:
        out[..., f] = c * a + s * b
        out[..., g] = -s * a + c * b
    return out


def reposition(k, p_old, p_new, base: float = 10000.0, style: str = "half",
               dtype: str = "bf16") -> np.ndarray:
    """Cache re-positioning, literal two-step form.

    [CacheFocus §2.3]: the inverse of a 2-D rotation is its transpose, so a key
    stored at position ``p_old`` is first un-rotated with ``R(p_old)^T`` and then
    rotated to its new position with ``R(p_new)``.  [InfoFlow §4.2] uses the same
    operation for global position reconstruction ``g(t) = Delta_i + p_i(t)``.
    The result is a cache tensor and is rounded to the cache dtype.

    ``k``: ``[..., N, H, D]``; ``p_old``, ``p_new``: positions ``[..., N]`` (all kv
    heads of a row share the row's position).
    """
    k = np.asarray(k, dtype=np.float64)
    po = np.asarray(p_old, dtype=np.float64)[..., None]
    pn = np.asarray(p_new, dtype=np.float64)[..., None]
    unrotated = rope_rotate(k, po, base, style, transpose=True)
    return round_to(rope_rotate(unrotated, pn, base, style), dtype)


# ---------------------------------------------------------------------------
# Query -> cache attention
# ---------------------------------------------------------------------------

def _kv_head(h: int, Hq: int, H: int) -> int:
    return h // (Hq // H)


def logits(q, k, scale: float) -> np.ndarray:
    """Scaled dot products ``l[b,h,j,t] = scale * q[b,j,h,:] . k[b,t,kv(h),:]``.

    [ACRE §2.1 Eq. 4] (``scale = 1/sqrt(d)``) and the query-to-L1 attention of
    [ACRE §2.4].  Returns ``[B][Hq][T][N]`` float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, T, Hq, D = q.shape
    H = k.shape[2]
    out = np.empty((B, Hq, T, k.shape[1]), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            out[b, h] = scale * (q[b, :, h, :] @ k[b, :, _kv_head(h, Hq, H), :].T)
    return out


def attention_weights(q, k, scale: float) -> np.ndarray:
    """Softmax of the query rows over every cached row of the instance.

    [ACRE §2.4]: ``A = softmax(Q_q K^T / sqrt(d))``.  Reading: the softmax runs
    over all N cached rows of one instance, with no mask and no query
    self-keys (every cached row precedes the query).  ``[B][Hq][T][N]``.
    """
    lg = logits(q, k, scale)
    e = np.exp(lg - lg.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def score(q, k, scale: float, unit_len: int = 1):
    """Row statistics and per-unit softmax partials of the query block.

    Definitions (from the softmax of [ACRE §2.1 Eq. 4]):

    * ``row_max[b,h,j] = max_t l[b,h,j,t]``
    * ``row_sum[b,h,j] = sum_t exp(l[b,h,j,t] - row_max[b,h,j])``
    * for units of ``unit_len`` consecutive cached rows, ``part[b,h,j,u] =
      (m_u, S_u)`` with ``m_u = max_{t in u} l`` and
      ``S_u = sum_{t in u} exp(l - m_u)``.

    Returns ``(row_max, row_sum, part)``; ``part`` is None when ``unit_len == 1``.
    """
    lg = logits(q, k, scale)
    row_max = lg.max(axis=-1)
    row_sum = np.exp(lg - row_max[..., None]).sum(axis=-1)
    part = None
    if unit_len > 1:
        B, Hq, T, N = lg.shape
        lu = lg.reshape(B, Hq, T, N // unit_len, unit_len)
        m_u = lu.max(axis=-1)
        s_u = np.exp(lu - m_u[..., None]).sum(axis=-1)
        part = np.stack([m_u, s_u], axis=-1)
    return row_max, row_sum, part


def combine_partials(part):
    """Row statistics recovered from per-unit partials (m_u, S_u).

    ``m = max_u m_u``; ``Z = sum_u S_u exp(m_u - m)`` -- the usual merge of
    softmax partial sums.  Returns ``(row_max, row_sum)``.
    """
    part = np.asarray(part, dtype=np.float64)
    m_u, s_u = part[..., 0], part[..., 1]
    m = m_u.max(axis=-1)
    return m, (s_u * np.exp(m_u - m[..., None])).sum(axis=-1)


def aggregate(q, k, v, scale: float, signal: str = "mass", unit_len: int = 1,
              group: int = 1) -> np.ndarray:
    """Per-unit relevance scores from the softmax-normalised attention.

    * "mass": ``S[g,u] = sum_{b in g} sum_h sum_j sum_{t in u} A[b,h,j,t]``.
      [ACRE §2.4 Eq. 15] pools A over heads and query tokens (a mean; the sum
      used here differs by the positive factor ``1/(Hq T)`` and ranks
      identically), [CacheFocus §2.4, footnote 3] accumulates the attention
      document-wise.
    * "vnorm": ``s[g,t] = sum_{b in g} sum_h sum_j A[b,h,j,t] * ||v[b,t,kv(h)]||_2``.
      [InfoFlow §4.2] scores token j by ``s_j = sum_i A_ij`` over the prompt
      rows, called an attention-norm signal; the definition of ``A_ij`` did not
      survive on the page.  Reading: attention weight times the L2 norm of the
      attended value row, summed over heads and query tokens.

    ``group`` consecutive instances (e.g. the layers whose scores are summed,
    [InfoFlow, Norm Layer Selection]) are added together.  Returns
    ``[B // group][N // unit_len]``.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, T, Hq, D = q.shape
    N, H = k.shape[1], k.shape[2]
    A = attention_weights(q, k, scale)
    per_token = np.zeros((B, N), dtype=np.float64)
    if signal == "vnorm":
        vn = np.linalg.norm(np.asarray(v, dtype=np.float64), axis=-1)   # [B][N][H]
    elif signal != "mass":
        raise ValueError(f"unknown signal {signal!r}")
    for h in range(Hq):
        a = A[:, h].sum(axis=1)                                          # over j
        if signal == "vnorm":
            a = a * vn[:, :, _kv_head(h, Hq, H)]
        per_token += a
    per_unit = per_token.reshape(B, N // unit_len, unit_len).sum(axis=-1)
    return per_unit.reshape(B // group, group, N // unit_len).sum(axis=1)


def acre_mean_pool(A) -> np.ndarray:
    """[ACRE §2.4 Eq. 15]: ``S = Pool_{dim=0,2}(A)`` for ``A`` in R^{h x m x t}.

    Takes the page's own axis order (heads, L1 entries, query tokens) and
    averages over heads and query tokens; returns ``S`` in R^m.
    """
    return np.asarray(A, dtype=np.float64).mean(axis=(0, 2))


# ---------------------------------------------------------------------------
# Selection
# ---------------------------------------------------------------------------

def topk(scores, k: int) -> np.ndarray:
    """Arg-top-k of each score row, returned in ascending index order.

    [ACRE §2.4 Eq. 16] ``I = argtop_k(S)``.  Reading for ties (silent on the
    pages): the order is score descending, then index ascending.  The kept set
    is listed in ascending index order, the order-preserving layout of
    [ACRE §2.4 Eq. 18-19].  ``scores``: ``[G][M]``; returns int64 ``[G][k]``.
    """
    s = np.asarray(scores, dtype=np.float64)
    G, M = s.shape
    k = max(0, min(int(k), M))
    out = np.empty((G, k), dtype=np.int64)
    idx = np.arange(M)
    for g in range(G):
        order = np.lexsort((idx, -s[g]))      # last key is primary
        out[g] = np.sort(order[:k])
    return out


# ---------------------------------------------------------------------------
# Gather / refill
# ---------------------------------------------------------------------------

def gather(k, v, idx, unit_len: int, idx_group: int = 1):
    """Copy the kept units' rows into a compact cache, kept units in order.

    [ACRE §2.4 Eq. 18-19] (refilled rows keep their order) and the final cache
    of [CacheFocus §2.4].  Instance ``b`` uses index row ``b // idx_group``; unit
    ``u`` is source rows ``[u*unit_len, (u+1)*unit_len)``.  Returns
    ``(k_out, v_out)`` shaped ``[B][k*unit_len][H][D]``.
    """
    k = np.asarray(k)
    v = np.asarray(v)
    idx = np.asarray(idx)
    B = k.shape[0]
    rows = [np.concatenate([np.arange(u * unit_len, (u + 1) * unit_len)
                            for u in idx[b // idx_group]]).astype(np.int64)
            if idx.shape[1] else np.zeros(0, np.int64) for b in range(B)]
    k_out = np.stack([k[b, rows[b]] for b in range(B)])
    v_out = np.stack([v[b, rows[b]] for b in range(B)])
    return k_out, v_out


def gather_aligned(k, idx, unit_len: int, p_old, align_base: int,
                   base: float = 10000.0, style: str = "half",
                   dtype: str = "bf16", idx_group: int = 1) -> np.ndarray:
    """Gather kept keys and re-position them to contiguous new positions.

    [CacheFocus §2.4-2.5]: after pruning, the remaining caches are re-positioned
    once more ("align": dynamic contiguous positions).  Reading: the r-th kept
    unit (ascending index order) takes positions
    ``align_base + r*unit_len + (0 .. unit_len-1)``.  ``p_old[b, t]`` is the
    position at which source row t is stored.  Literal two-step re-positioning
    from the stored key, then rounding to the cache dtype.
    """
    k = np.asarray(k, dtype=np.float64)
    idx = np.asarray(idx)
    p_old = np.asarray(p_old, dtype=np.float64)
    B = k.shape[0]
    outs = []
    for b in range(B):
        sel = idx[b // idx_group]
        parts = []
        for r, u in enumerate(sel):
            rows = np.arange(u * unit_len, (u + 1) * unit_len)
            p_new = align_base + r * unit_len + np.arange(unit_len)
            parts.append(reposition(k[b, rows], p_old[b, rows], p_new, base, style, dtype))
        outs.append(np.concatenate(parts) if parts else np.zeros((0,) + k.shape[2:]))
    return np.stack(outs)


def refill_nested(l1, l2, idx, l: int) -> np.ndarray:
    """The refilled bi-layer cache in the nested order of [ACRE §2.4 Eq. 18-19].

    L1 entry j (0-based here) proxies L2 rows ``[j*l, (j+1)*l)`` ([ACRE §2.3
    Eq. 11-12]).  Walking the L1 entries in order, a selected entry is preceded
    by its L2 block; an unselected one stands alone.  ``l1``: ``[m][...]``,
    ``l2``: ``[n][...]``, ``idx``: selected L1 indices.  Returns
    ``[m + len(idx)*l][...]``.
    """
    l1 = np.asarray(l1)
    l2 = np.asarray(l2)
    chosen = set(int(j) for j in np.asarray(idx).ravel())
    rows = []
    for j in range(l1.shape[0]):
        if j in chosen:
            rows.extend(l2[j * l:(j + 1) * l])
        rows.append(l1[j])
    return np.stack(rows)


# ---------------------------------------------------------------------------
# Final attention pass
# ---------------------------------------------------------------------------

def decode_attention(q, segments: Sequence, scale: float):
    """One attention pass of the query rows over the compact cache.

    [ACRE §2.1 Eq. 4] ``softmax(Q K^T / sqrt(d)) V`` over the concatenation of
    ``segments`` (each a ``(k, v)`` pair ``[B][N_s][H][D]``), with no mask.
    Returns ``(o, lse)``: ``o`` is ``[B][T][Hq][D]``; ``lse[b,h,j]`` is the natural
    log of ``sum_t exp(l[b,h,j,t])``.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.concatenate([np.asarray(s[0], dtype=np.float64) for s in segments], axis=1)
    V = np.concatenate([np.asarray(s[1], dtype=np.float64) for s in segments], axis=1)
    B, T, Hq, D = q.shape
    H = K.shape[2]
    lg = logits(q, K, scale)
    m = lg.max(axis=-1)
    e = np.exp(lg - m[..., None])
    Z = e.sum(axis=-1)
    A = e / Z[..., None]
    o = np.empty((B, T, Hq, V.shape[-1]), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            o[b, :, h, :] = A[b, h] @ V[b, :, _kv_head(h, Hq, H), :]
    return o, m + np.log(Z)


def index_causal_attention(q, k, v, pos, scale: float):
    """Attention of selected tokens to the context under a causal constraint
    ([InfoFlow §4.2] KV recomputation: a selected token is run at its global
    position, so it attends to every context row up to and including its own;
    [InfoFlow §8]: an index-based causal pattern, neither dense nor strictly
    causal).

    ``q``: ``[B][S][Hq][D]``, the queries of the S selected tokens;
    ``pos``: ``[B][S]``, their positions in the context; ``k``, ``v``:
    ``[B][N][H][D]``.  Row (b, i, h) attends to keys ``0 .. pos[b][i]``
    (clipped to N - 1); a negative position attends to nothing and gives a
    zero row and lse = -inf.  Returns ``(o [B][S][Hq][D], lse [B][Hq][S])``
    with lse the natural log of the row's sum of exp(logit).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.int64)
    B, S, Hq, D = q.shape
    N, H = k.shape[1], k.shape[2]
    o = np.zeros((B, S, Hq, v.shape[-1]), dtype=np.float64)
    lse = np.full((B, Hq, S), -np.inf, dtype=np.float64)
    for b in range(B):
        for i in range(S):
            n = min(int(pos[b, i]), N - 1) + 1
            if n <= 0:
                continue
            for h in range(Hq):
                g = _kv_head(h, Hq, H)
                lg = scale * (k[b, :n, g, :] @ q[b, i, h, :])
                m = lg.max()
                e = np.exp(lg - m)
                o[b, i, h] = (e @ v[b, :n, g, :]) / e.sum()
                lse[b, h, i] = m + np.log(e.sum())
    return o, lse


# ---------------------------------------------------------------------------
# Host-side arithmetic of the three methods
# ---------------------------------------------------------------------------

def acre_k(W: int, m: int, eta: int, l: int) -> int:
    """[ACRE §2.4 Eq. 17]: ``k = floor(min(W - m, eta) / l)``.

    Reading: clamped at 0 when the L1 cache alone exceeds the working window
    (``m > W``), where the formula would go negative.
    """
    return max(0, math.floor(min(W - m, eta) / l))


def cf_group_size(L: int, l_c: int) -> int:
    """[CacheFocus §2.3.1]: at most ``L / l_C`` caches get unique positions."""
    return L // l_c


def cf_reuse_count(k: int, L: int, l_c: int) -> int:
    """[CacheFocus §2.3.1]: number of reuses ``N_reuse`` for k caches.

    The formula did not survive on the page; reading: ``ceil(k / (L // l_C))``,
    the fewest groups of at most ``L / l_C`` caches that hold all k.
    """
    return -(-k // cf_group_size(L, l_c))


def cf_doc_starts(n_docs: int, doc_len: int, L: int) -> np.ndarray:
    """Start position of each document cache under adaptive re-positioning.

    [CacheFocus §2.3.1]: the caches are split into ``N_reuse`` groups and the
    caches within a group get sequential positions.  Reading: groups are runs
    of ``L // doc_len`` consecutive documents, so document u starts at
    ``(u mod (L // doc_len)) * doc_len``.
    """
    G = cf_group_size(L, doc_len)
    return np.array([(u % G) * doc_len for u in range(n_docs)], dtype=np.int64)


def cf_k_prune(k: int, k_finish: int, L: int, n: int) -> float:
    """[CacheFocus App. C]: caches pruned per pruning layer,
    ``(k - k_finish) / (L / n)`` (L layers, pruning every n-th layer)."""
    return (k - k_finish) / (L / n)


def cf_prune_layers(L: int, n: int) -> list:
    """[CacheFocus §2.4]: a pruning operation runs at every n-th layer of the
    pre-fill.  With layers counted from 0 these are layers n-1, 2n-1, ...;
    ``L // n`` of them."""
    return [l for l in range(L) if (l + 1) % n == 0]


def cf_keep_schedule(k: int, k_finish: int, L: int, n: int) -> list:
    """Caches left after each pruning layer.

    [CacheFocus App. C]: each pruning layer removes ``k_prune = (k - k_finish) /
    (L / n)`` caches, so that ``k_finish`` remain after the last one (worked
    example: L=28, n=4, k=40, k_finish=5 gives 5).  Reading where that is not a
    whole number: with P = ``L // n`` pruning layers, ``k - floor(p (k - k_finish)
    / P)`` caches remain after the p-th, which removes exactly k_prune each time
    when it is whole, leaves k_finish after the last, and otherwise spreads the
    remainder so that no two pruning layers differ by more than one cache.
    """
    P = len(cf_prune_layers(L, n))
    return [k - (p * (k - k_finish)) // P for p in range(1, P + 1)]


def cf_progressive_prune(q_layers, k_layers, doc_len: int, scale: float, n: int,
                         k_finish: int, window: int, base: float = 10000.0,
                         style: str = "half", dtype: str = "bf16",
                         score_after_last_prune: bool = True) -> dict:
    """Layer-Adaptive Cache Pruning of [CacheFocus §2.4] for one request.

    ``q_layers``: ``[L][T][Hq][D]``, the query block of every layer (already at
    its positions); ``k_layers``: ``[L][k * doc_len][H][D]``, the k retrieved
    document caches of every layer, document i in rows ``[i*doc_len,
    (i+1)*doc_len)``, each stored at document-local positions ``0 .. doc_len-1``
    ([CacheFocus §2.2]: every document cache is pre-computed on its own).

    At every layer l:

    1. the caches of the current cache IDs (ascending: the retrieval order) are
       concatenated and re-positioned: the j-th gets the start position of
       slot j under adaptive re-positioning (:func:`cf_doc_starts` with the
       positional range ``window``, [CacheFocus §2.3.1]), token t of it goes
       from position t to ``start_j + t`` (:func:`reposition`);
    2. the layer's query attends the whole concatenation (:func:`attention_weights`);
    3. the attention is accumulated document-wise ([CacheFocus §2.4 fn. 3]:
       summed over heads, query tokens and the document's tokens) and added to
       the document's running total.  Reading: the relevance S a pruning layer
       uses is this total over all layers so far (the footnote's progressive
       accumulation), not the pruning layer's own attention alone;
    4. at a pruning layer (:func:`cf_prune_layers`), only the
       :func:`cf_keep_schedule` count of caches with the largest totals stay
       (ties: smaller cache ID), kept in ascending ID order.

    After the last layer the remaining IDs are listed two ways ([CacheFocus
    §2.5]): "align", ascending ID (positions follow continuity), and "sort",
    by total with the most relevant last, i.e. nearest the query that follows
    the caches (reading of the attention-guided allocation, after [CacheFocus
    §2.5]'s point that relevant documents near the query help).  Layers after
    the last pruning layer only change the "sort" order; with
    ``score_after_last_prune=False`` they are not scored.

    Returns a dict: ``ids`` (IDs present at each layer), ``mass`` (each
    layer's document-wise attention, in the order of ``ids``), ``total``
    (running totals after each layer, same order), ``starts`` (slot start
    positions at each layer), ``final_align``, ``final_sort`` and
    ``final_total`` (totals of ``final_align``).
    """
    q_layers = np.asarray(q_layers, dtype=np.float64)
    k_layers = np.asarray(k_layers, dtype=np.float64)
    L = q_layers.shape[0]
    k = k_layers.shape[1] // doc_len
    prune_at = dict(zip(cf_prune_layers(L, n), cf_keep_schedule(k, k_finish, L, n)))
    last_prune = max(prune_at) if prune_at else -1
    ids = np.arange(k, dtype=np.int64)
    total = np.zeros(k, dtype=np.float64)          # by cache ID
    out = {"ids": [], "mass": [], "total": [], "starts": []}
    for l in range(L):
        m = ids.size
        if l > last_prune and not score_after_last_prune:
            break
        rows = (ids[:, None] * doc_len + np.arange(doc_len)[None, :]).reshape(-1)
        starts = cf_doc_starts(m, doc_len, window)
        p_old = np.tile(np.arange(doc_len), m)
        p_new = np.repeat(starts, doc_len) + p_old
        k_rep = reposition(k_layers[l][rows], p_old, p_new, base, style, dtype)
        A = attention_weights(q_layers[l][None], k_rep[None], scale)[0]     # [Hq][T][m*doc_len]
        mass = A.reshape(A.shape[0], A.shape[1], m, doc_len).sum(axis=(0, 1, 3))
        total[ids] += mass
        out["ids"].append(ids.copy())
        out["mass"].append(mass)
        out["total"].append(total[ids].copy())
        out["starts"].append(starts)
        if l in prune_at:
            keep = topk(total[ids][None], prune_at[l])[0]     # positions in the current list
            ids = ids[keep]
    out["final_align"] = ids.copy()
    by_relevance = np.lexsort((ids, -total[ids]))             # most relevant first
    out["final_sort"] = ids[by_relevance[::-1]].copy()
    out["final_total"] = total[ids].copy()
    return out


def take(src, idx) -> np.ndarray:
    """Composition of index lists, ``out[g][j] = src[g][idx[g][j]]``
    ([CacheFocus §2.4]: the cache IDs left after a pruning layer are the kept
    positions of the current ID list).  ``-1`` where an index is outside
    ``[0, m)``."""
    src = np.asarray(src, dtype=np.int64)
    idx = np.asarray(idx, dtype=np.int64)
    out = np.full(idx.shape, -1, dtype=np.int64)
    for g in range(idx.shape[0]):
        ok = (idx[g] >= 0) & (idx[g] < src.shape[1])
        out[g, ok] = src[g, idx[g, ok]]
    return out


def order(scores, idx, descending: bool = True) -> np.ndarray:
    """The given indices of each row listed by score ([CacheFocus §2.5]
    attention-guided "sort" allocation).  Order: score descending, then index
    ascending (the tie rule of :func:`topk`), then position in the given list;
    ``descending=False`` lists the exact reverse (most relevant last).  An
    index outside ``[0, M)`` ranks below every valid one."""
    s = np.asarray(scores, dtype=np.float64)
    idx = np.asarray(idx, dtype=np.int64)
    out = np.empty_like(idx)
    for g in range(idx.shape[0]):
        ok = (idx[g] >= 0) & (idx[g] < s.shape[1])
        sc = np.where(ok, s[g, np.clip(idx[g], 0, s.shape[1] - 1)], 0.0)
        pos = np.arange(idx.shape[1])
        rank = np.lexsort((pos, idx[g], -sc, ~ok))        # last key is primary
        out[g] = idx[g, rank] if descending else idx[g, rank[::-1]]
    return out


def cf_final_cache(k_layers, v_layers, final_ids, doc_len: int, start: int = 0,
                   base: float = 10000.0, style: str = "half", dtype: str = "bf16"):
    """The combined final cache of [CacheFocus §2.4]: for every layer, the
    caches of ``final_ids`` (in that order) concatenated and re-positioned to
    contiguous positions ``start + r * doc_len + t`` (slot r, token t; §2.5
    assigns the remaining caches new consecutive positions).  Keys stored at
    document-local positions; values are copied.  Returns ``(K, V)`` of shape
    ``[L][len(final_ids) * doc_len][H][D]``."""
    k_layers = np.asarray(k_layers, dtype=np.float64)
    v_layers = np.asarray(v_layers, dtype=np.float64)
    ids = np.asarray(final_ids, dtype=np.int64)
    rows = (ids[:, None] * doc_len + np.arange(doc_len)[None, :]).reshape(-1)
    p_old = np.tile(np.arange(doc_len), ids.size)
    p_new = start + np.arange(ids.size * doc_len)
    K = np.stack([reposition(k_layers[l][rows], p_old, p_new, base, style, dtype)
                  for l in range(k_layers.shape[0])])
    return K, v_layers[:, rows].copy()


def if_chunk_offsets(chunk_lens: Iterable[int]) -> np.ndarray:
    """[InfoFlow §4.2] ``Delta_i``: global start of chunk i, the total length of
    the chunks before it in the concatenated order."""
    lens = np.asarray(list(chunk_lens), dtype=np.int64)
    return np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)


def if_global_positions(chunk_lens: Iterable[int]) -> np.ndarray:
    """[InfoFlow §4.1-4.2]: token t of chunk i, stored at chunk-local position
    ``p_i(t)`` (0 .. |C_i|-1), gets the global position ``g(t) = Delta_i + p_i(t)``."""
    lens = list(chunk_lens)
    off = if_chunk_offsets(lens)
    return np.concatenate([off[i] + np.arange(n) for i, n in enumerate(lens)]).astype(np.int64)


def if_chunk_fractions(sel, chunk_lens: Sequence[int]) -> np.ndarray:
    """[InfoFlow §4.3]: ``r_i = |S^(1) ∩ C_i| / |C_i|``, the share of chunk i's
    tokens in the first-stage selection.  Chunks lie back to back in storage
    (chunk i covers the rows after chunks 0..i-1).  ``sel``: selected row
    indices ``[G][k]``; returns ``[G][n_chunks]``."""
    sel = np.asarray(sel, dtype=np.int64)
    lens = np.asarray(list(chunk_lens), dtype=np.int64)
    bounds = np.concatenate([[0], np.cumsum(lens)])
    out = np.zeros((sel.shape[0], lens.size), dtype=np.float64)
    for g in range(sel.shape[0]):
        chunk = np.searchsorted(bounds, sel[g], side="right") - 1
        for c in chunk:
            out[g, c] += 1.0
    return out / lens[None, :]


def if_reorder(r) -> np.ndarray:
    """[InfoFlow §4.3, §6.2]: the new chunk order, informative chunks nearest
    the prompt (which follows the context).  Reading for the order: chunks
    ranked by (r descending, index ascending), the top-k order, and placed so
    that rank 0 comes last.  Returns ``order[G][n]``: ``order[g][p]`` is the
    chunk at position p of the new concatenation."""
    r = np.asarray(r, dtype=np.float64)
    out = np.empty(r.shape, dtype=np.int64)
    idx = np.arange(r.shape[1])
    for g in range(r.shape[0]):
        ranked = np.lexsort((idx, -r[g]))            # most informative first
        out[g] = ranked[::-1]
    return out


def if_reordered_offsets(order, chunk_lens: Sequence[int]) -> np.ndarray:
    """[InfoFlow §4.3]: GLOBAL positions rebuilt for the new concatenated order
    (``g(t) = Delta_i + p_i(t)`` with ``Delta_i`` the length of the chunks now
    before chunk i).  Returns ``Delta[G][n]`` indexed by the original chunk."""
    order = np.asarray(order, dtype=np.int64)
    lens = np.asarray(list(chunk_lens), dtype=np.int64)
    out = np.empty(order.shape, dtype=np.int64)
    for g in range(order.shape[0]):
        acc = 0
        for c in order[g]:
            out[g, c] = acc
            acc += lens[c]
    return out


def if_two_stage(q, k, v, chunk_lens: Sequence[int], scale: float, budget: int,
                 group: int = 1, base: float = 10000.0, style: str = "half",
                 dtype: str = "bf16", signal: str = "vnorm") -> dict:
    """Two-stage selection with chunk reordering, [InfoFlow §4.3] and [InfoFlow
    §5.1]'s choice of geometries.

    1. First stage in the HL-TP geometry: the chunks keep their chunk-local
       positions (the stored keys, no re-positioning) and the prompt sits at
       its global position (the query block as given).  Token scores
       (:func:`aggregate`, summed over ``group`` consecutive instances) and the
       budget ``budget`` (:func:`topk`) give S^(1).
    2. ``r_i`` (:func:`if_chunk_fractions`), the new order (:func:`if_reorder`)
       and the GLOBAL positions of that order (:func:`if_reordered_offsets`).
    3. Second stage: the keys re-positioned from their local positions to
       ``Delta_i + p_i(t)`` (:func:`reposition`), scored again, and the same
       budget selected: S^(2), as row indices of the stored cache.

    ``k``, ``v``: ``[B][N][H][D]`` at chunk-local positions; ``q``: ``[B][T][Hq][D]``.
    """
    k = np.asarray(k, dtype=np.float64)
    lens = list(chunk_lens)
    s1 = aggregate(q, k, v, scale, signal, 1, group)
    sel1 = topk(s1, budget)
    r = if_chunk_fractions(sel1, lens)
    order = if_reorder(r)
    delta = if_reordered_offsets(order, lens)
    local = np.concatenate([np.arange(n) for n in lens]).astype(np.int64)
    chunk_of = np.repeat(np.arange(len(lens)), lens)
    B = k.shape[0]
    G = B // group
    p_new = np.stack([local + delta[b // group][chunk_of] for b in range(B)])
    k2 = reposition(k, np.broadcast_to(local, (B, local.size)), p_new, base, style, dtype)
    s2 = aggregate(q, k2, v, scale, signal, 1, group)
    sel2 = topk(s2, budget)
    assert s2.shape[0] == G
    return {"score1": s1, "sel1": sel1, "r": r, "order": order, "delta": delta,
            "k_rep": k2, "score2": s2, "sel2": sel2}


def if_budget(n_tokens: int, ratio: str = "0.15") -> int:
    """[InfoFlow §6.1]: a fixed recomputation ratio (15%) of the context
    tokens.  Reading: ``floor(ratio * n_tokens)``, in exact rational arithmetic."""
    return int(math.floor(Fraction(ratio) * n_tokens))
