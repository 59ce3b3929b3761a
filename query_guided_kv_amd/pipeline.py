"""The selection path of each workload as a sequence of library calls.

``run(w, inp)`` executes re-position -> score -> aggregate -> top-k ->
gather/refill -> decode attention for one input batch on the GPU and returns
every intermediate (device tensors), so that each call can be checked on its
own.  Only argument preparation happens here; all tensor work is done by the
HIP kernels behind :mod:`query_guided_kv_amd.kvsel`.
"""

from __future__ import annotations

import torch

from . import host
from . import kvsel as K


def reposition_deltas(w, device) -> tuple:
    """(delta tensor, re-positioning unit length) of workload ``w``, or (None, 0).
    Keys are stored at unit-local positions 0..len-1."""
    if w.reposition == "none":
        return None, 0
    if w.reposition == "global":            # InfoFlow KV §4.2, GLOBAL geometry
        L = int(w.plants["chunk_len"])
        return host.delta_tensor(host.chunk_offsets([L] * (w.N // L)), device), L
    if w.reposition == "contiguous":        # chunks placed back to back
        L = w.unit_len
        return host.delta_tensor(host.chunk_offsets([L] * (w.N // L)), device), L
    if w.reposition == "reuse_window":      # CacheFocus §2.3.1
        L = w.unit_len
        return host.delta_tensor(host.reuse_window_starts(w.N // L, L, w.window), device), L
    raise ValueError(w.reposition)


def run(w, inp: dict, row_stats: bool = True) -> dict:
    q, k, v = inp["q"], inp["k"], inp["v"]
    dev = k.device
    out = {}
    delta, L = reposition_deltas(w, dev)
    k_score = k
    if delta is not None:
        k_score = K.reposition(k, delta, L, rope_base=w.rope_base, style=w.rope_style)
        out["k_rep"] = k_score
    if w.unit_len > 1 and w.signal == "mass":
        rm, rs, part = K.score(q, k_score, w.unit_len, w.scale, row_stats=row_stats, partials=True)
        out.update(row_max=rm, row_sum=rs, part=part)
        out["unit_score"] = K.aggregate(w.unit_len, w.group, "mass", part=part, row_max=rm,
                                        row_sum=rs, k=k_score, scale=w.scale)
    else:
        rm, rs, _ = K.score(q, k_score, w.unit_len, w.scale, row_stats=True, partials=False)
        out.update(row_max=rm, row_sum=rs)
        out["unit_score"] = K.aggregate(w.unit_len, w.group, w.signal, q=q, k=k_score, v=v,
                                        row_max=rm, row_sum=rs, scale=w.scale)
    out["idx"] = K.topk(out["unit_score"], w.k)
    if not w.decode:
        return out
    if w.refill_interval:                   # ACRE: L1 entry j -> its L2 block
        gk, gv = K.gather(inp["l2_k"], inp["l2_v"], out["idx"], w.refill_interval, w.group)
        segs = [(k, v), (gk, gv)]
    elif w.align:                           # CacheFocus "align": contiguous final slots
        gk, gv = K.gather(k, v, out["idx"], w.unit_len, w.group, align_base=0,
                          rope_base=w.rope_base, style=w.rope_style)
        segs = [(gk, gv)]
    else:
        gk, gv = K.gather(k_score, v, out["idx"], w.unit_len, w.group)
        segs = [(gk, gv)]
    out["k_gather"], out["v_gather"] = gk, gv
    out["o"], out["lse"] = K.decode_attn(q, segs, w.scale)
    return out


def run_nested_refill(w, inp: dict, idx: torch.Tensor):
    """ACRE Eq. 18-19 nested layout: each kept L1 entry preceded by its L2 block."""
    return K.gather(inp["l2_k"], inp["l2_v"], idx, w.refill_interval, w.group,
                    proxy_k=inp["k"], proxy_v=inp["v"])


class Path:
    """One workload's hot path with every argument prepared once.

    ``path(q)`` runs re-position -> score -> aggregate -> top-k -> gather ->
    decode attention for one query block with the fewest launches each step
    needs (chunk workloads: one scoring kernel that emits only the per-unit
    partials, row statistics derived inside the aggregate call).  ``marks``
    maps a stage name to a (start, end) pair of torch.cuda.Event recorded on
    the launch stream around that stage.

    Outputs and workspaces are allocated by the first call and reused by every
    later one: a step allocates nothing after the first, so a loop of steps
    makes no allocator calls and a step captured as a HIP graph replays into
    the same buffers.  The returned tensors are those buffers: the next call
    overwrites them (clone what must outlive it).
    """

    STAGES = ("score", "aggregate", "topk", "gather", "decode", "gather_decode")

    def __init__(self, w, inp: dict):
        self.w = w
        self.k, self.v = inp["k"], inp["v"]
        self.l2 = (inp.get("l2_k"), inp.get("l2_v"))
        dev = self.k.device
        self.delta, self.delta_len = reposition_deltas(w, dev)
        # re-positioned keys are kept where later steps read them; the aligned
        # gather re-positions from the stored keys instead
        keep = self.delta is not None and not w.align
        self.k_rep = torch.empty_like(self.k) if keep else None
        self.chunk = w.unit_len > 1 and w.signal == "mass"
        # refill and attention are one call where one kernel does both (it
        # reads each kept row once); the aligned gather re-positions on the way
        rows = (w.Hq // w.H) * w.T
        one_pass = (w.dtype == "bf16" and w.D == 128 and 1 <= rows <= 8
                    and w.H in (1, 2, 4, 8))
        split = w.decode and (w.align or not one_pass)
        self.split = split
        self.stages = tuple(s for s in self.STAGES
                            if (s not in ("gather", "decode") or split)
                            and (s != "gather_decode" or (w.decode and not split)))
        self.buf = {}                                   # outputs kept across calls
        self.ws = {s: K.Workspace() for s in ("score", "aggregate", "decode")}
        # Launch plans: each call site's library calls, as marshalled on its
        # first run, are made again as they are while the query block (its
        # address and shape) and the stream stay the same: every other
        # argument is this object's own input or buffer.  A short step is
        # otherwise bound by the host time of the argument checks.
        self.plans = {}

    def _keep(self, *pairs):
        """Record the outputs a call allocated (first call) or filled."""
        for name, t in pairs:
            if t is not None:
                self.buf[name] = t

    def __call__(self, q: torch.Tensor, marks: dict = None) -> dict:
        w = self.w
        ev = marks or {}
        b = self.buf
        key = (q.data_ptr(), tuple(q.shape), torch.cuda.current_stream(q.device).cuda_stream)

        def mark(stage, i):
            pair = ev.get(stage)
            if pair is not None:
                pair[i].record()

        def planned(site, fn):
            plan = self.plans.get(site)
            if plan is not None and plan[0] == key:
                K.replay(plan[1])
                return plan[2]
            with K.Recording() as calls:
                res = fn()
            self.plans[site] = (key, calls, res)
            return res

        out = {}
        k_score = self.k if self.k_rep is None else self.k_rep

        def score(stats: bool, partials: bool):
            outs = dict(rm_out=b.get("row_max"), rs_out=b.get("row_sum"),
                        part_out=b.get("part"), ws=self.ws["score"])
            # re-positioning happens inside the scoring call (one read of K)
            if self.delta is None:
                res = K.score(q, self.k, w.unit_len, w.scale, row_stats=stats,
                              partials=partials, **outs)
            else:
                res = K.score_reposition(q, self.k, self.delta, self.delta_len, w.unit_len,
                                         k_out=self.k_rep, scale=w.scale, row_stats=stats,
                                         partials=partials, rope_base=w.rope_base,
                                         style=w.rope_style, **outs)
            self._keep(*zip(("row_max", "row_sum", "part"), res))
            return res

        if self.k_rep is not None:
            out["k_rep"] = self.k_rep
        if self.chunk:
            mark("score", 0)
            _, _, part = planned("score", lambda: score(False, True))
            mark("score", 1)
            mark("aggregate", 0)
            out["unit_score"] = planned("aggregate", lambda: K.aggregate(
                w.unit_len, w.group, "mass", part=part, cache_shape=tuple(k_score.shape), q=q,
                out=b.get("unit_score"), ws=self.ws["aggregate"]))
            mark("aggregate", 1)
        else:
            mark("score", 0)
            rm, rs, _ = planned("score", lambda: score(True, False))
            mark("score", 1)
            mark("aggregate", 0)
            out["unit_score"] = planned("aggregate", lambda: K.aggregate(
                w.unit_len, w.group, w.signal, q=q, k=k_score, v=self.v, row_max=rm, row_sum=rs,
                scale=w.scale, out=b.get("unit_score"), ws=self.ws["aggregate"]))
            mark("aggregate", 1)
        mark("topk", 0)
        out["idx"] = planned("topk", lambda: K.topk(out["unit_score"], w.k, idx_out=b.get("idx")))
        mark("topk", 1)
        self._keep(("unit_score", out["unit_score"]), ("idx", out["idx"]))
        if not w.decode:
            return out
        gouts = dict(k_out=b.get("k_gather"), v_out=b.get("v_gather"))
        douts = dict(out=b.get("o"), lse_out=b.get("lse"), ws=self.ws["decode"])
        if self.split:
            # the copy (re-positioned for "align"), then attention over it
            mark("gather", 0)
            if w.align:
                gk, gv = planned("gather", lambda: K.gather(
                    self.k, self.v, out["idx"], w.unit_len, w.group, align_base=0,
                    rope_base=w.rope_base, style=w.rope_style, **gouts))
            elif w.refill_interval:     # ACRE: L1 entry j -> its L2 block
                gk, gv = planned("gather", lambda: K.gather(
                    self.l2[0], self.l2[1], out["idx"], w.refill_interval, w.group, **gouts))
            else:
                gk, gv = planned("gather", lambda: K.gather(
                    k_score, self.v, out["idx"], w.unit_len, w.group, **gouts))
            mark("gather", 1)
            mark("decode", 0)
            segs = [(self.k, self.v), (gk, gv)] if w.refill_interval else [(gk, gv)]
            out["o"], out["lse"] = planned("decode", lambda: K.decode_attn(q, segs, w.scale,
                                                                           **douts))
            mark("decode", 1)
        else:
            # refill and attention in one pass over the kept rows
            mark("gather_decode", 0)
            if w.refill_interval:       # ACRE: L1 entry j -> its L2 block, L1 kept as a segment
                gk, gv, o, lse = planned("gather_decode", lambda: K.gather_decode(
                    q, self.l2[0], self.l2[1], out["idx"], w.refill_interval, w.group,
                    extra=[(self.k, self.v)], scale=w.scale, **gouts, **douts))
            else:
                gk, gv, o, lse = planned("gather_decode", lambda: K.gather_decode(
                    q, k_score, self.v, out["idx"], w.unit_len, w.group, scale=w.scale,
                    **gouts, **douts))
            mark("gather_decode", 1)
            out["o"], out["lse"] = o, lse
        out["k_gather"], out["v_gather"] = gk, gv
        self._keep(("k_gather", gk), ("v_gather", gv), ("o", out["o"]), ("lse", out["lse"]))
        return out


class PrunePath:
    """CacheFocus layer-adaptive cache pruning (§2.4) for a batch of requests,
    then the final re-positioning (§2.4-2.5) and one decode attention pass.

    Caches are a request-major store ``[requests * layers][n_docs * doc_len][H][D]``
    of document caches at document-local positions; ``q_layers`` is
    ``[layers][requests][T][Hq][D]``.  Per layer, one call scores every
    request's current documents in place, each re-positioned to its slot
    (:func:`kvsel.score_units` on the layer's strided view of the store), and one
    call adds the document-wise attention to the running totals; after every
    n-th layer a top-k keeps the scheduled number of documents (with their
    totals) and a take composes the kept positions with the current IDs.  The
    survivors are listed in ID order ("align") or by total, most relevant last
    ("sort"), and a gather re-positions them to consecutive slots for every
    layer.  Every step is a library call; this class only sequences them.
    """

    STAGES = ("select", "final_gather", "decode")

    def __init__(self, w, inp: dict):
        self.w = w
        R, L, U = w.requests, w.layers, w.unit_len
        self.k, self.v = inp["k"], inp["v"]
        dev = self.k.device
        self.n_docs = w.N // U
        # one layer's caches of all requests: a strided view of the store
        self.k_layer = self.k.view(R, L, w.N, w.H, w.D)
        self.prune_at = dict(zip(host.prune_layers(L, w.prune_every),
                                 host.keep_schedule(self.n_docs, w.k, L, w.prune_every)))
        final = list(self.prune_at.values())[-1] if self.prune_at else self.n_docs
        if final != w.k:
            raise ValueError(f"the pruning schedule ends at {final} documents, not k={w.k}")
        lengths = {self.n_docs, *self.prune_at.values()}
        self.delta = {m: host.delta_tensor(host.reuse_window_starts(m, U, w.window), dev)
                      for m in lengths}
        self.ids0 = torch.arange(self.n_docs, dtype=torch.int32, device=dev).repeat(R, 1)
        self.iota = torch.arange(w.k, dtype=torch.int32, device=dev).repeat(R, 1)
        last = max(self.prune_at) if self.prune_at else -1
        # layers after the last pruning layer only change the "sort" order
        self.n_scored = L if w.allocation == "sort" else last + 1
        self.stages = self.STAGES if w.decode else self.STAGES[:2]

    def select(self, q_layers: torch.Tensor, trace: list = None, score_marks: list = None):
        """Run the layer loop; returns (final IDs [R][k] in allocation order,
        their totals in ID order).  ``trace`` collects (ids, totals) per layer;
        ``score_marks`` holds a (start, end) event pair per scored layer,
        recorded around its scoring call."""
        w = self.w
        U = w.unit_len
        ids, total = self.ids0, None
        for l in range(self.n_scored):
            m = ids.shape[1]
            if score_marks is not None:
                score_marks[l][0].record()
            _, _, part = K.score_units(q_layers[l], self.k_layer[:, l], ids, U,
                                       delta=self.delta[m], scale=w.scale, row_stats=False,
                                       partials=True, rope_base=w.rope_base, style=w.rope_style)
            if score_marks is not None:
                score_marks[l][1].record()
            if total is None:
                total = torch.empty((ids.shape[0], m), dtype=torch.float32, device=ids.device)
            K.aggregate(U, 1, "mass", part=part, cache_shape=(ids.shape[0], m * U, w.H, w.D),
                        q=q_layers[l], out=total, accumulate=l > 0)
            if trace is not None:
                trace.append((ids.clone(), total.clone()))
            keep = self.prune_at.get(l)
            if keep is not None:
                pos, total = K.topk(total, keep, values=True)
                ids = K.take(ids, pos)
        final = ids
        if w.allocation == "sort":
            final = K.take(ids, K.order(total, self.iota, descending=False))
        return final, total

    def __call__(self, q_layers: torch.Tensor, q_dec: torch.Tensor = None, marks: dict = None,
                 trace: list = None) -> dict:
        w = self.w
        ev = marks or {}

        def mark(stage, i):
            pair = ev.get(stage)
            if pair is not None:
                pair[i].record()

        out = {}
        mark("select", 0)
        out["idx"], out["total"] = self.select(q_layers, trace, ev.get("score_layers"))
        mark("select", 1)
        mark("final_gather", 0)
        out["k_gather"], out["v_gather"] = K.gather(self.k, self.v, out["idx"], w.unit_len,
                                                    w.layers, align_base=0,
                                                    rope_base=w.rope_base, style=w.rope_style)
        mark("final_gather", 1)
        if w.decode and q_dec is not None:
            mark("decode", 0)
            out["o"], out["lse"] = K.decode_attn(q_dec, [(out["k_gather"], out["v_gather"])],
                                                 w.scale)
            mark("decode", 1)
        return out


class ReorderPath:
    """InfoFlow two-stage selection with chunk reordering (§4.3, with the
    geometries of §5.1), as library calls:

    1. first stage on the stored chunk-local keys (HL-TP: the query block as
       given, at the prompt's global position): score, token scores summed
       over the layers of a selection, top-k;
    2. the share r_i of each chunk's tokens in that selection
       (:func:`kvsel.unit_fractions`), the chunks listed with the most
       informative last (:func:`kvsel.order`), and each chunk's start in that
       order (:func:`kvsel.slot_starts`);
    3. second stage with the keys re-positioned to those GLOBAL starts (fused
       into scoring; the re-positioned keys are kept for the token scores),
       and the same budget selected again.
    """

    STAGES = ("score1", "aggregate1", "topk1", "reorder", "score2", "aggregate2", "topk2")

    def __init__(self, w, inp: dict):
        self.w = w
        self.k, self.v = inp["k"], inp["v"]
        dev = self.k.device
        self.chunk_len = int(w.plants["chunk_len"])
        self.n_chunks = w.N // self.chunk_len
        G = w.B // w.group
        self.iota = torch.arange(self.n_chunks, dtype=torch.int32, device=dev).repeat(G, 1)
        self.k_rep = torch.empty_like(self.k)
        self.stages = self.STAGES

    def __call__(self, q: torch.Tensor, marks: dict = None) -> dict:
        w = self.w
        ev = marks or {}

        def mark(stage, i):
            pair = ev.get(stage)
            if pair is not None:
                pair[i].record()

        def select(k, tag, delta=None):
            mark("score" + tag, 0)
            if delta is None:
                rm, rs, _ = K.score(q, k, 1, w.scale, row_stats=True, partials=False)
                kk = k
            else:
                rm, rs, _ = K.score_reposition(q, k, delta, self.chunk_len, 1, k_out=self.k_rep,
                                               scale=w.scale, row_stats=True, partials=False,
                                               rope_base=w.rope_base, style=w.rope_style)
                kk = self.k_rep
            mark("score" + tag, 1)
            mark("aggregate" + tag, 0)
            s = K.aggregate(1, w.group, w.signal, q=q, k=kk, v=self.v, row_max=rm, row_sum=rs,
                            scale=w.scale)
            mark("aggregate" + tag, 1)
            mark("topk" + tag, 0)
            idx = K.topk(s, w.k)
            mark("topk" + tag, 1)
            return s, idx

        out = {}
        out["score1"], out["sel1"] = select(self.k, "1")
        mark("reorder", 0)
        out["r"] = K.unit_fractions(out["sel1"], self.chunk_len, self.n_chunks)
        out["order"] = K.order(out["r"], self.iota, descending=False)
        out["delta"] = K.slot_starts(out["order"], self.chunk_len, rep=w.group)
        mark("reorder", 1)
        out["score2"], out["sel2"] = select(self.k, "2", out["delta"])
        out["k_rep"] = self.k_rep
        # the product of the path: the final selection and the chunk layout
        out["idx"], out["unit_score"] = out["sel2"], out["score2"]
        return out


class RecomputePath:
    """The recomputation attention of the selected tokens ([InfoFlow §4.2]):
    every selected token's query attends to the context rows up to its own
    position (:func:`kvsel.index_attn`), for every layer."""

    STAGES = ("recompute",)

    def __init__(self, w, inp: dict):
        self.w = w
        self.k, self.v, self.pos = inp["k"], inp["v"], inp["pos"]
        self.stages = self.STAGES

    def __call__(self, q_sel: torch.Tensor, marks: dict = None) -> dict:
        ev = marks or {}
        pair = ev.get("recompute")
        if pair is not None:
            pair[0].record()
        o, lse = K.index_attn(q_sel, self.k, self.v, self.pos, self.w.scale)
        if pair is not None:
            pair[1].record()
        return {"o": o, "lse": lse}


def make_path(w, inp: dict):
    """The launch sequence of workload ``w``."""
    if w.recipe == "cachefocus":
        return PrunePath(w, inp)
    if w.reorder:
        return ReorderPath(w, inp)
    if w.recompute:
        return RecomputePath(w, inp)
    return Path(w, inp)
