"""Oracle side of each workload: the selection path run step by step on the CPU.

Test infrastructure: calls only ``oracle`` and the seeded inputs.  Each stage's
output is kept so that every library call can be checked on its own as well as
end to end.
"""

from __future__ import annotations

import numpy as np
import torch

from . import kvsel_oracle as O


def to64(t) -> np.ndarray:
    """Exact float64 copy of a (bf16 / fp32) torch tensor; numpy arrays pass
    through as float64."""
    if isinstance(t, np.ndarray):
        return t.astype(np.float64, copy=False)
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def positions(w, n_instances: int):
    """(p_old, p_new) per cached row for the workload's re-positioning, or None.

    Keys are stored at unit-local positions 0..unit_len-1 (chunk-wise prefill,
    [InfoFlow §4.1]; per-document caches, [CacheFocus §2.2]).
    """
    if w.reposition == "none":
        return None
    L = w.plants.get("chunk_len", w.unit_len) if w.reposition == "global" else w.unit_len
    n_units = w.N // L
    p_old = np.tile(np.arange(L), n_units)
    if w.reposition in ("contiguous", "global"):
        p_new = O.if_global_positions([L] * n_units)            # g(t) = Delta_i + p_i(t)
    elif w.reposition == "reuse_window":
        starts = O.cf_doc_starts(n_units, L, w.window)
        p_new = np.repeat(starts, L) + p_old
    else:
        raise ValueError(w.reposition)
    return (np.broadcast_to(p_old, (n_instances, w.N)),
            np.broadcast_to(p_new, (n_instances, w.N)))


def margin(scores_row: np.ndarray, k: int) -> float:
    """Relative gap at the top-k cut: (s_(k) - s_(k+1)) / s_(k)."""
    s = np.sort(np.asarray(scores_row, np.float64))[::-1]
    if k <= 0 or k >= s.size:
        return np.inf
    return (s[k - 1] - s[k]) / s[k - 1]


def run(w, inp: dict, instances=None) -> dict:
    """Oracle path for workload ``w`` on inputs ``inp`` (from ``synth.generate``).

    ``instances``: optional list of instance indices to evaluate (selection
    groups of size 1 only); default all.
    """
    out = {}
    B = w.B
    sel = list(range(B)) if instances is None else list(instances)
    q = to64(inp["q"])[sel]
    k = to64(inp["k"])[sel]
    v = to64(inp["v"])[sel]
    pos = positions(w, len(sel))
    if pos is not None:
        k_rep = O.reposition(k, pos[0], pos[1], w.rope_base, w.rope_style, w.dtype)
        out["k_rep"] = k_rep
    else:
        k_rep = k
    group = w.group if instances is None else 1
    out["row_max"], out["row_sum"], out["part"] = O.score(q, k_rep, w.scale, w.unit_len)
    out["unit_score"] = O.aggregate(q, k_rep, v, w.scale, w.signal, w.unit_len, group)
    out["idx"] = O.topk(out["unit_score"], w.k)
    out["margin"] = [margin(r, w.k) for r in out["unit_score"]]
    if not w.decode:
        return out
    if w.refill_interval:
        l2k = to64(inp["l2_k"])[sel]
        l2v = to64(inp["l2_v"])[sel]
        gk, gv = O.gather(l2k, l2v, out["idx"], w.refill_interval)
        segs = [(k, v), (gk, gv)]
    elif w.align:
        gk = O.gather_aligned(k, out["idx"], w.unit_len, pos[0], 0,
                              w.rope_base, w.rope_style, w.dtype)
        _, gv = O.gather(k, v, out["idx"], w.unit_len)
        segs = [(gk, gv)]
    else:
        gk, gv = O.gather(k_rep, v, out["idx"], w.unit_len)
        segs = [(gk, gv)]
    out["k_gather"], out["v_gather"] = gk, gv
    out["o"], out["lse"] = O.decode_attention(q, segs, w.scale)
    return out
