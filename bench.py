#!/usr/bin/env python3
"""Throughput of query-guided KV selection on one MI355X.

One step is one pass of the whole hot path -- re-position (where the workload
has it) -> score -> aggregate -> top-k -> gather/refill -> decode attention --
over one batch of synthetic input that is already resident in HBM.  The
default workload is batched serving: 16 requests x 8 layers = 128 independent
caches of 131,072 tokens (GQA 32/8, head dim 128, bf16; 68.7 GB of K and V);
each step draws a fresh one-token query per (request, layer), keeps the top 64
chunks of 256 tokens, gathers them and runs decode attention over the 16,384
kept rows.

Prints one JSON line:
  value       cached KV token-rows scored and selected per second (B x N per
              step / step time);
  roofline    the dominant (longest) stage's kernel: its algorithmic bytes (or
              flops, where it runs on the matrix cores above the bf16 ridge)
              per launch over its average launch time (HIP events on its
              launch stream), against MI355X's 8 TB/s (or 2.5 PFLOP/s bf16);
              traffic is the HBM bytes the counters measured for that kernel
              (null when no measurement matches the source);
  cpu_baseline  the fp64 CPU oracle on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""

from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, vendor figure
MFMA_BF16_TFLOPS = 2500.0       # MI355X dense bf16 matrix peak, vendor figure
HOST_LINK_GBPS = 64.0           # PCIe 5.0 x16, one direction (MI355X's host link)
MFMA_RIDGE = MFMA_BF16_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)   # flop per byte
DEFAULT_WORKLOAD = "serving_16req_8l_128k"
PROFILES = os.path.join(ROOT, "profiles")
# kernel sources whose hash keys a stored counter measurement
_C = "query_guided_kv_amd/csrc/"
KERNEL_SOURCES = {
    "score_stream_kernel": [_C + "score.hip", _C + "common.h"],
    "score_tile_kernel": [_C + "score.hip", _C + "common.h"],
    "score_mfma_kernel": [_C + "score_mfma.hip", _C + "mfma.h", _C + "common.h"],
    "agg_mfma_kernel": [_C + "aggregate_mfma.hip", _C + "mfma.h", _C + "common.h"],
    "agg_token_kernel": [_C + "aggregate.hip", _C + "common.h"],
    "topk_reg_kernel": [_C + "topk.hip", _C + "common.h"],
    "topk_stream_kernel": [_C + "topk.hip", _C + "common.h"],
    "gather_kernel": [_C + "gather.hip", _C + "common.h"],
    "decode_stream_kernel": [_C + "decode.hip", _C + "mfma.h", _C + "common.h"],
    "decode_mfma_kernel": [_C + "decode.hip", _C + "mfma.h", _C + "common.h"],
    "decode_tile_kernel": [_C + "decode.hip", _C + "common.h"],
    "index_attn_kernel": [_C + "index_attn.hip", _C + "mfma.h", _C + "common.h"],
    "order_kernel": [_C + "topk.hip", _C + "common.h"],
    "decode_merge_kernel": [_C + "decode.hip"],
}

# Stages of the selection proper (the rest of a step refills and attends).
SELECTION_STAGES = ("score", "aggregate", "topk", "score1", "aggregate1", "topk1", "reorder",
                    "score2", "aggregate2", "topk2", "select")

# The decode calls run split-K: a pass over the keys, then the merge of the
# splits.  Their stage is timed as one call, so its roofline names both kernels.
MERGE = "+decode_merge_kernel"


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_hash(kernel: str) -> str:
    """Hash of the sources of a kernel, or of every kernel of an 'a+b' call."""
    h = hashlib.sha256()
    rels = []
    for k in kernel.split("+"):
        rels += [r for r in KERNEL_SOURCES[k] if r not in rels]
    for rel in rels:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def elem_bytes(w) -> int:
    return 2 if w.dtype == "bf16" else 4


def one_pass_decode(w) -> bool:
    """True where refill and decode attention run as one kernel (the streaming
    decode reads each kept row through the index, writes it to the compact
    cache and attends to it): bf16, head dim 128, 1, 2, 4 or 8 kv heads and
    1 to 8 query rows per kv head."""
    rows = (w.Hq // w.H) * w.T
    return w.dtype == "bf16" and w.D == 128 and 1 <= rows <= 8 and w.H in (1, 2, 4, 8)


def mfma_shape(w) -> bool:
    """Shapes whose scoring runs on the matrix cores."""
    return w.dtype == "bf16" and (w.Hq // w.H) * w.T >= 16


def decode_kernel(w, rows: int) -> str:
    """The kernel of a plain (not gathering) decode pass with `rows` query rows
    per kv head: the matrix cores from 5 rows (bf16), the streaming kernel
    below that where it applies, else the tile kernel."""
    stream = w.dtype == "bf16" and w.D == 128 and 1 <= rows <= 8 and w.H in (1, 2, 4, 8)
    if w.dtype == "bf16" and rows >= 5:
        return "decode_mfma_kernel"
    return "decode_stream_kernel" if stream else "decode_tile_kernel"


def stage_work(w) -> dict:
    """Algorithmic work of one step, per stage: ``(bytes, flops)``.

    Bytes count every distinct region once (the scored keys read once, the
    values once if their norm is needed, the re-positioned keys written once
    where they are a product, the kept rows read once and the compact cache
    written once); re-reads are implementation cost.  Flops are the products
    the stage needs: 2 per multiply-add of the query-key logits (scoring) and
    of both attention products (decode); re-computation is not counted."""
    row = w.H * w.D * elem_bytes(w)
    rows = w.B * w.N
    qk = 2 * w.B * w.Hq * w.T * w.N * w.D          # one pass of query x cached keys
    out = {"score": [rows * row, qk]}
    if w.reposition != "none" and not w.align:
        out["score"][0] += rows * row               # re-positioned keys written (a product)
    out["aggregate"] = [rows * row if w.signal == "vnorm" else 0, 0]   # values for their norms
    out["topk"] = [(w.B // w.group) * w.M * 4, 0]
    if w.decode:
        per_unit = w.refill_interval if w.refill_interval else w.unit_len
        kept_rows = w.k * per_unit
        keys = kept_rows + (w.N if w.refill_interval else 0)   # ACRE attends L1 + refilled rows
        gather = [2 * 2 * w.B * kept_rows * row, 0]            # K and V, read and written
        decode = [(w.B * w.N * row if w.refill_interval else 0),  # L1 values (keys: scoring)
                  4 * w.B * w.Hq * w.T * keys * w.D]
        if one_pass_decode(w) and not w.align:                 # one call: refill + attention
            out["gather_decode"] = [gather[0] + decode[0], decode[1]]
        else:
            out["gather"], out["decode"] = gather, decode
    return {s: tuple(v) for s, v in out.items()}


def prune_scored_units(w) -> int:
    """Documents scored per request over the layer loop of a pruning workload
    (every layer scores the documents still present; layers after the last
    pruning layer are scored only for the "sort" order)."""
    from query_guided_kv_amd import host
    prune = dict(zip(host.prune_layers(w.layers, w.prune_every),
                     host.keep_schedule(w.M, w.k, w.layers, w.prune_every)))
    last = max(prune) if prune else -1
    n_scored = w.layers if w.allocation == "sort" else last + 1
    m, total = w.M, 0
    for l in range(n_scored):
        total += m
        m = prune.get(l, m)
    return total


def prune_stage_work(w) -> dict:
    """(bytes, flops) per stage of the layer-wise pruning path: the select loop
    reads the present documents' keys once per scored layer; the final gather
    reads and writes the survivors' K and V for every layer; the decode pass
    attends them (its reads are the gather's writes, counted there)."""
    row = w.H * w.D * elem_bytes(w)
    scored_rows = w.requests * prune_scored_units(w) * w.unit_len
    kept_rows = w.B * w.k * w.unit_len
    return {"select": (scored_rows * row, 2 * scored_rows * (w.Hq // w.H) * w.T * w.H * w.D),
            "final_gather": (2 * 2 * kept_rows * row, 0),
            "decode": (0, 4 * w.B * w.Hq * 1 * w.k * w.unit_len * w.D)}


def reorder_stage_work(w) -> dict:
    """(bytes, flops) per stage of the two-stage selection: each stage reads
    the keys once (the second also writes the re-positioned keys, a product it
    scores from) and the values once for their norms; re-reads are
    implementation cost."""
    row = w.H * w.D * elem_bytes(w)
    rows = w.B * w.N
    qk = 2 * w.B * w.Hq * w.T * w.N * w.D
    top = (w.B // w.group) * w.M * 4
    return {"score1": (rows * row, qk), "aggregate1": (rows * row, 0), "topk1": (top, 0),
            "reorder": (0, 0),
            "score2": (2 * rows * row, qk), "aggregate2": (rows * row, 0), "topk2": (top, 0)}


def recompute_stage_work(w, pos) -> dict:
    """(bytes, flops) of the recomputation attention: every selected row reads
    keys 0 .. pos (2 flops per multiply-add of q.k and of p.v); the context's K
    and V are read once (re-reads by other row blocks are implementation cost)."""
    import numpy as np
    p = np.minimum(np.asarray(pos.cpu(), np.int64), w.N - 1) + 1
    keys = int(np.clip(p, 0, None).sum())                 # over instances and rows
    row = w.H * w.D * elem_bytes(w)
    return {"recompute": (2 * w.B * w.N * row, 4 * w.Hq * w.D * keys)}


def stage_bound(stage: str, w, work) -> tuple:
    """(bound, algorithmic quantity, peak, unit) of a stage: the matrix cores
    where the stage runs on them and its flops per algorithmic byte exceed the
    bf16 ridge of MI355X (2.5 PFLOP/s over 8 TB/s = 312.5), else HBM."""
    nbytes, flops = work
    if w.l2_host and stage == "gather":
        # the kept L2 rows cross the host link once (half of the gather's
        # algorithmic bytes: they are then written to HBM)
        return "host_link", nbytes / 2 / 1e9, HOST_LINK_GBPS, "GB/s"
    rows = (w.Hq // w.H) * (1 if (w.recipe == "cachefocus" and stage == "decode") else w.T)
    on_mfma = w.dtype == "bf16" and rows >= 16 and stage in ("score", "decode", "select",
                                                             "score1", "score2", "recompute")
    if on_mfma and flops > MFMA_RIDGE * max(nbytes, 1):
        return "mfma", flops / 1e12, MFMA_BF16_TFLOPS, "TFLOP/s"
    return "hbm", nbytes / 1e9, HBM_PEAK_GBPS, "GB/s"


def kernel_of(stage: str, w) -> str:
    """Name of the kernel that carries a stage's work for workload w."""
    if w.recipe == "cachefocus":
        return {"select": "score_mfma_kernel" if mfma_shape(w) else "score_stream_kernel",
                "final_gather": "gather_kernel",
                "decode": decode_kernel(w, w.Hq // w.H) + MERGE}[stage]   # one decode token
    if stage == "recompute":
        return "index_attn_kernel"
    if w.reorder and stage not in ("score", "aggregate", "topk"):
        stage = {"score1": "score", "score2": "score", "aggregate1": "aggregate",
                 "aggregate2": "aggregate", "topk1": "topk", "topk2": "topk"}.get(stage, stage)
        if stage == "reorder":
            return "order_kernel"
    rows = (w.Hq // w.H) * w.T
    stream = w.dtype == "bf16" and w.D == 128 and rows in (1, 2, 4, 8)
    mfma = mfma_shape(w)
    return {"score": "score_stream_kernel" if stream else
                     "score_mfma_kernel" if mfma else "score_tile_kernel",
            "aggregate": "agg_mfma_kernel" if mfma else "agg_token_kernel",
            "topk": "topk_reg_kernel" if w.N // w.unit_len <= 65536 else "topk_stream_kernel",
            "gather": "gather_kernel",
            "decode": decode_kernel(w, rows) + MERGE,
            "gather_decode": "decode_stream_kernel" + MERGE}[stage]


def stored_traffic(kernel: str, workload: str):
    """HBM bytes per launch from a committed counter summary, or None when
    there is none for this kernel's current source."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.lstrip().startswith("#"):
                k, v = (s.strip() for s in line.split("=", 1))
                vals[k] = v
    if vals.get("source_hash") != source_hash(kernel):
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def make_queries(w, inp, n: int, seed: int, device):
    from query_guided_kv_amd import synth
    if w.recipe == "serving":
        return [synth.serving_queries(w, inp["topic"], seed, s, device) for s in range(n)]
    return [inp["q"]] * n


def cpu_baseline_prune(w, inp, threads: int, layers: int = 8) -> dict:
    """The fp64 oracle's layer loop on request 0, first ``layers`` layers
    (two pruning layers at n = 4) with ``threads`` BLAS threads; rate in scored
    token-rows per second."""
    from threadpoolctl import threadpool_limits
    from oracle import kvsel_oracle as O
    from oracle import pipeline as OP

    L = min(layers, w.layers)
    q = OP.to64(inp["q"][:L, 0])
    k = OP.to64(inp["k"][:L])
    with threadpool_limits(limits=threads):
        t0 = time.perf_counter()
        res = O.cf_progressive_prune(q, k, w.unit_len, w.scale, w.prune_every, w.k, w.window,
                                     w.rope_base, w.rope_style, w.dtype)
        elapsed = time.perf_counter() - t0
    rows = sum(ids.size for ids in res["ids"]) * w.unit_len
    log(f"cpu oracle ({threads} threads): {L} layers of request 0 in {elapsed:.1f} s")
    return {"value": rows / elapsed, "unit": "token-rows/s", "cores": threads, "kind": "oracle",
            "sample": f"request 0, layers 0-{L - 1} of the pruning loop ({rows} scored "
                      f"token-rows; fp64 numpy, {threads} BLAS threads), {elapsed:.1f} s"}


def cpu_baseline_reorder(w, inp, threads: int) -> dict:
    """The fp64 oracle's two-stage selection on one layer's share (instance 0
    as a selection of its own, same budget); rate in scored token-rows per
    second (two passes over the cache)."""
    from threadpoolctl import threadpool_limits
    from oracle import kvsel_oracle as O
    from oracle import pipeline as OP

    sub = {key: OP.to64(inp[key][0:1]) for key in ("q", "k", "v")}
    lens = [int(w.plants["chunk_len"])] * (w.N // int(w.plants["chunk_len"]))
    with threadpool_limits(limits=threads):
        t0 = time.perf_counter()
        O.if_two_stage(sub["q"], sub["k"], sub["v"], lens, w.scale, w.k, 1, w.rope_base,
                       w.rope_style, w.dtype, w.signal)
        elapsed = time.perf_counter() - t0
    rows = 2 * w.N
    log(f"cpu oracle ({threads} threads): two-stage selection of instance 0 in {elapsed:.1f} s")
    return {"value": rows / elapsed, "unit": "token-rows/s", "cores": threads, "kind": "oracle",
            "sample": f"instance 0 of {w.B} as its own selection (2 x {w.N} scored token-rows; "
                      f"fp64 numpy, {threads} BLAS threads), {elapsed:.1f} s"}


def cpu_baseline_recompute(w, inp, threads: int, rows: int = 64) -> dict:
    """The fp64 oracle on a sample of the recomputation: ``rows`` selected
    tokens of layer 0 (every head); rate in attended (row, key) pairs per
    second, the unit the GPU line reports."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import kvsel_oracle as O
    from oracle import pipeline as OP

    S = inp["pos"].shape[1]
    pick = np.linspace(0, S - 1, rows).astype(np.int64)
    q = OP.to64(inp["q_sel"][0:1])[:, pick]
    pos = inp["pos"][0:1].cpu().numpy()[:, pick]
    k, v = OP.to64(inp["k"][0:1]), OP.to64(inp["v"][0:1])
    with threadpool_limits(limits=threads):
        t0 = time.perf_counter()
        O.index_causal_attention(q, k, v, pos, w.scale)
        elapsed = time.perf_counter() - t0
    pairs = int((np.minimum(pos, w.N - 1) + 1).sum())
    log(f"cpu oracle ({threads} threads): {rows} recomputed rows in {elapsed:.1f} s")
    return {"value": pairs / elapsed, "unit": "token-rows/s", "cores": threads, "kind": "oracle",
            "sample": f"{rows} of {S} selected tokens of layer 0, every head ({pairs} attended "
                      f"context rows; fp64 numpy, {threads} BLAS threads), {elapsed:.1f} s"}


def host_cpu() -> dict:
    """The host the oracle ran on: CPU model, logical CPUs, CPUs this process may use."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "cpu_count": os.cpu_count(),
            "affinity": len(os.sched_getaffinity(0))}


def cpu_baseline(w, inp, threads: int, budget_s: float = 8.0, max_instances: int = 16) -> dict:
    """Time the fp64 oracle on whole instances of the workload (inputs copied to
    host memory first, outside the timed region) with ``threads`` BLAS
    threads, until ``budget_s`` seconds or ``max_instances`` instances."""
    from threadpoolctl import threadpool_limits
    from oracle import pipeline as OP

    if w.group > 1:
        # one selection spans `group` instances (e.g. the layers of InfoFlow):
        # time one instance's share of it and scale by the instance count
        wi = w.scaled(B=1, group=1)
    else:
        wi = w.scaled(B=1, requests=1)
    done, elapsed = 0, 0.0
    with threadpool_limits(limits=threads):
        while done < min(max_instances, w.B) and elapsed < budget_s:
            b = done
            sub = {key: OP.to64(inp[key][b:b + 1]) for key in ("q", "k", "v")}
            for key in ("l2_k", "l2_v"):
                if key in inp:
                    sub[key] = OP.to64(inp[key][b:b + 1])
            t0 = time.perf_counter()
            OP.run(wi, sub)
            elapsed += time.perf_counter() - t0
            done += 1
            log(f"cpu oracle ({threads} threads): instance {b} done, {elapsed:.1f} s so far")
    rows = done * w.N
    return {"value": rows / elapsed, "unit": "token-rows/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} of {w.B} instances ({w.N} cached rows each, whole path, "
                      f"fp64 numpy, {threads} BLAS threads), {elapsed:.1f} s"}


def cpu_baselines(w, inp, prune: bool) -> dict:
    """The oracle with BLAS threads set to the CPUs this process may use, and
    single-threaded beside it (numpy's elementwise work runs on one thread
    either way)."""
    threads = len(os.sched_getaffinity(0))
    leg = (lambda t: cpu_baseline_prune(w, inp, t)) if prune else \
        (lambda t: cpu_baseline_reorder(w, inp, t)) if w.reorder else \
        (lambda t: cpu_baseline_recompute(w, inp, t)) if w.recompute else \
        (lambda t: cpu_baseline(w, inp, t))
    res = leg(threads)
    res["single_thread"] = leg(1) if threads > 1 else dict(res)
    res["host"] = host_cpu()
    return res


def step_timeline(start, stop, marks, first: str, last: str, step_ms: list,
                  host_ms: list) -> dict:
    """Where the GPU clock of the staged pass (the timed steps run again with
    an event pair around every stage) went outside the steps' own spans: from
    the pass's start event to step 0's first stage (lead), between one step's
    last stage and the next step's first (gaps), and after the last step
    (tail); with the spread of the step spans and the host time each step's
    launches took (a host slower than the GPU leaves gaps)."""
    gaps = [marks[i][last][1].elapsed_time(marks[i + 1][first][0])
            for i in range(len(marks) - 1)]
    spans = sorted(step_ms)
    p90 = spans[min(len(spans) - 1, int(round(0.9 * (len(spans) - 1))))]
    return {"lead_ms": start.elapsed_time(marks[0][first][0]),
            "gap_ms_total": sum(gaps), "gap_ms_max": max(gaps, default=0.0),
            "tail_ms": marks[-1][last][1].elapsed_time(stop),
            "step_span_ms": {"mean": statistics.mean(spans), "median": statistics.median(spans),
                             "p90": p90, "max": spans[-1]},
            "host_launch_ms": {"mean": statistics.mean(host_ms), "max": max(host_ms)}}


def time_graph(step, feed, steps: int, warmup: int, rows: int) -> dict:
    """The step captured once as a HIP graph (torch.cuda.graph) and replayed
    ``args.steps`` times between events: what a serving loop that launches the
    whole path at once would see.  ``step()`` runs the path on its static
    inputs; ``feed(i)`` (or None) copies step i's fresh inputs into them (the
    serving workload's new queries), on the same stream, inside the timed
    region."""
    import torch
    side = torch.cuda.Stream()                     # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for i in range(max(warmup, 1)):
        if feed is not None:
            feed(i)
        graph.replay()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        if feed is not None:
            feed(warmup + i)
        graph.replay()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    log(f"{steps} graph replays: {ms:.4f} ms per step")
    return {"ms_per_step": ms, "value": rows / (ms * 1e-3),
            "inputs_copied_per_step": feed is not None}


def device_copy_rate(dev) -> float:
    """The device's own copy rate: 1 GiB read + 1 GiB written per copy, timed
    on the GPU clock (the path's HBM rate is also given against it)."""
    import torch
    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(5):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    return 5 * 2 * (1 << 30) / (a.elapsed_time(b) * 1e-3) / 1e9


def host_link_rate(dev) -> dict:
    """The host link's DMA rate: 1 GiB pinned host -> device, on the GPU clock."""
    import torch
    src = torch.empty(1 << 28, dtype=torch.float32, pin_memory=True)
    dst = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    for _ in range(2):
        dst.copy_(src, non_blocking=True)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(5):
        dst.copy_(src, non_blocking=True)
    b.record()
    torch.cuda.synchronize()
    return {"dma_copy_GBps": 5 * (1 << 30) / (a.elapsed_time(b) * 1e-3) / 1e9,
            "peak_GBps": HOST_LINK_GBPS}


def measure(w, seed: int, steps: int, warmup: int, graph: bool, copy_GBps: float, dev) -> tuple:
    """Time ``steps`` steps of workload ``w`` (after ``warmup`` untimed ones)
    between events on the launch stream, with a (start, end) event pair around
    every stage; returns (result dict, inputs, rows per step)."""
    import torch
    from query_guided_kv_amd import pipeline, synth

    log(f"workload {w.name}: B={w.B} N={w.N} Hq/H={w.Hq}/{w.H} D={w.D} T={w.T} {w.dtype}")
    host_link = None
    if w.l2_host:
        host_link = host_link_rate(dev)
        log(f"host link: pinned -> device copy at {host_link['dma_copy_GBps']:.1f} GB/s")
    t0 = time.perf_counter()
    inp = synth.generate(w, seed, dev)
    torch.cuda.synchronize()
    log(f"inputs generated in {time.perf_counter() - t0:.1f} s")
    prune = w.recipe == "cachefocus"
    path = pipeline.make_path(w, inp)
    queries = None
    if prune:
        step = lambda i, m=None: path(inp["q"], inp["q_dec"], m)
    elif w.recompute:
        step = lambda i, m=None: path(inp["q_sel"], m)
    else:
        queries = make_queries(w, inp, warmup + steps, seed, dev)
        step = lambda i, m=None: path(queries[i], m)

    # no garbage collection inside the warm-up and timed regions: a collection
    # pauses the host for tens of ms, and one that falls before the first
    # timed launches leaves the GPU idle (the queue is still empty)
    gc.collect()
    gc.disable()
    try:
        for i in range(warmup):
            step(i)
        torch.cuda.synchronize()
        log(f"{warmup} warm-up steps done")

        marks = [{s: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for s in path.stages} for _ in range(steps)]
        if prune:   # the scorer's launches inside the layer loop, one pair per scored layer
            for mk in marks:
                mk["score_layers"] = [(torch.cuda.Event(enable_timing=True),
                                       torch.cuda.Event(enable_timing=True))
                                      for _ in range(path.n_scored)]
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        # create every event now (torch makes the HIP event on its first
        # record), so that the timed region only records them
        for mk in marks:
            for pairs in mk.values():
                for pair in (pairs if isinstance(pairs, list) else [pairs]):
                    for e in pair:
                        e.record()
        start.record()
        stop.record()
        torch.cuda.synchronize()
        # the timed steps alone: no event between the region's start and stop
        # (an event costs the GPU about 3 us, a fifth of a 0.12 ms step)
        wall0 = time.perf_counter()
        start.record()
        for i in range(steps):
            step(warmup + i)
        stop.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        total_ms = start.elapsed_time(stop)
        # the same steps again with an event pair around every stage: stage
        # times (the roofline's launch durations), step spans and the timeline
        start2, stop2 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start2.record()
        stop2.record()
        torch.cuda.synchronize()
        host_ms = []
        start2.record()
        for i in range(steps):
            h0 = time.perf_counter()
            step(warmup + i, marks[i])
            host_ms.append((time.perf_counter() - h0) * 1e3)
        stop2.record()
        torch.cuda.synchronize()
    finally:
        gc.enable()
    ms_step = total_ms / steps
    staged_ms = start2.elapsed_time(stop2) / steps
    log(f"{steps} timed steps: {total_ms:.2f} ms on the GPU clock, {wall * 1e3:.2f} ms wall; "
        f"with stage events {staged_ms * steps:.2f} ms")

    work = (prune_stage_work(w) if prune else reorder_stage_work(w) if w.reorder
            else recompute_stage_work(w, inp["pos"]) if w.recompute else stage_work(w))
    stage_ms = {s: statistics.mean(m[s][0].elapsed_time(m[s][1]) for m in marks)
                for s in path.stages}
    # per-step times from the first stage's start to the last stage's end
    first, last = path.stages[0], path.stages[-1]
    step_ms = [m[first][0].elapsed_time(m[last][1]) for m in marks]
    timeline = step_timeline(start2, stop2, marks, first, last, step_ms, host_ms)
    timeline["ms_per_step_with_stage_events"] = staged_ms
    log(f"timeline: lead {timeline['lead_ms']:.3f} ms, gaps {timeline['gap_ms_total']:.3f} ms "
        f"(max {timeline['gap_ms_max']:.3f}), tail {timeline['tail_ms']:.3f} ms, "
        f"host launch {timeline['host_launch_ms']['mean']:.3f} ms/step "
        f"(max {timeline['host_launch_ms']['max']:.3f})")
    dom = max(path.stages, key=lambda s: stage_ms[s])     # the stage that takes longest
    dom_ms = stage_ms[dom]
    bound, quantity, peak, unit = stage_bound(dom, w, work[dom])
    launches = 1
    if prune and dom == "select":
        # the layer loop's bytes are the scorer's: time its launches alone
        # (the aggregates, top-ks and takes between them are excluded)
        dom_ms = statistics.mean(sum(a.elapsed_time(b) for a, b in m["score_layers"])
                                 for m in marks)
        launches = path.n_scored
        stage_ms["select_scoring"] = dom_ms
    achieved = quantity / (dom_ms * 1e-3)
    kernel = kernel_of(dom, w)
    # token-rows scored per step: every cached row once, or for the pruning
    # loop the rows of the documents present at each scored layer
    rows = (w.requests * prune_scored_units(w) * w.unit_len if prune
            else 2 * w.B * w.N if w.reorder
            else work["recompute"][1] // (4 * w.Hq * w.D) if w.recompute else w.B * w.N)
    path_bytes = sum(b for b, _ in work.values())
    result = {
        "value": rows / (ms_step * 1e-3),
        "ms_per_step": ms_step,
        "ms_per_step_median": statistics.median(step_ms),
        "dtype": w.dtype,
        "config": dict({"workload": w.name, "instances": w.B, "cached_rows_per_instance": w.N,
                        "q_heads": w.Hq, "kv_heads": w.H, "head_dim": w.D,
                        "query_tokens": w.T, "unit_len": w.unit_len, "kept_units": w.k,
                        "seed": seed},
                       **({"requests": w.requests, "layers": w.layers,
                           "prune_every": w.prune_every, "allocation": w.allocation,
                           "scored_rows_per_step": rows} if prune else {})),
        "roofline": {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
                     "frac": achieved / peak, "traffic": stored_traffic(kernel, w.name),
                     "kernel": kernel, "stage": dom,
                     "algorithmic_bytes_per_launch": work[dom][0] / launches,
                     "algorithmic_flops_per_launch": work[dom][1] / launches,
                     "launches_per_step": launches, "avg_launch_ms": dom_ms / launches},
        "path_hbm": {"algorithmic_bytes_per_step": path_bytes,
                     "achieved_GBps": path_bytes / (ms_step * 1e-3) / 1e9,
                     "frac": path_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                     "device_copy_GBps": copy_GBps,
                     "frac_of_device_copy": path_bytes / (ms_step * 1e-3) / 1e9 / copy_GBps},
        "stages_ms": stage_ms,
        "timeline": timeline,
    }
    # selection alone (re-position, score, aggregate, top-k; both stages and the
    # reordering of a two-stage selection; the pruning loop), beside the full path
    sel = [s for s in path.stages if s in SELECTION_STAGES]
    if sel:
        sel_ms = sum(stage_ms[s] for s in sel)
        result["selection"] = {"stages": sel, "ms_per_step": sel_ms,
                               "value": rows / (sel_ms * 1e-3), "unit": "token-rows/s"}
    if w.refill_interval:
        # every kept L1 entry stands for refill_interval L2 tokens
        result["covered"] = {"value": w.B * w.N * w.refill_interval / (ms_step * 1e-3),
                             "unit": "L2 token-rows/s", "l2_tokens_per_l1_entry": w.refill_interval}
    if host_link is not None:
        result["host_link"] = host_link
    if graph:
        if prune:
            result["graph"] = time_graph(lambda: path(inp["q"], inp["q_dec"]), None, steps,
                                         warmup, rows)
        elif w.recompute:
            result["graph"] = time_graph(lambda: path(inp["q_sel"]), None, steps, warmup, rows)
        elif w.recipe != "serving":
            result["graph"] = time_graph(lambda: path(inp["q"]), None, steps, warmup, rows)
        else:
            # the captured step reads a static query block; each replay is
            # preceded by a copy of that step's fresh queries into it
            static_q = queries[0].clone()
            result["graph"] = time_graph(lambda: path(static_q),
                                         lambda i: static_q.copy_(queries[i % len(queries)]),
                                         steps, warmup, rows)
    del path
    return result, inp, rows


# Measured beside the default line in the same run (steps timed, one entry
# each under "also"): the other workloads of the configurations, then the
# layer-wise pruning loop, the two-stage selection with reordering, the refill
# from host-resident L2 and the recompute attention of the selected tokens.
ALSO = (("acre_bilayer_l1_16k_l2_128k", 200), ("llama2_7b_32docs_x512", 200),
        ("infoflow_32l_64x1024", 30), ("cachefocus_qwen2_28l_40docs_x512", 10),
        ("infoflow_reorder_32l_64x1024", 10), ("acre_bilayer_host_l2_l1_16k_l2_128k", 50),
        ("infoflow_recompute_32l_64x1024", 3))


def also_entry(res: dict) -> dict:
    """The summary of one extra workload in the bench line."""
    keep = ("value", "ms_per_step", "dtype", "roofline", "stages_ms", "selection", "covered",
            "host_link", "graph")
    out = {k: res[k] for k in keep if k in res}
    # the staged pass (an event pair around every stage): its mean and median
    # per-step span include the events' own cost, a fifth of a 0.12 ms step
    out["staged_pass_ms_per_step"] = res["timeline"]["ms_per_step_with_stage_events"]
    out["staged_pass_ms_per_step_median"] = res["ms_per_step_median"]
    out["workload"] = res["config"]["workload"]
    out["unit"] = "token-rows/s"
    out["path_hbm_frac"] = res["path_hbm"]["frac"]
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-also", action="store_true",
                    help="skip the other workloads measured beside the default one")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 1 GiB streaming kernel (counter scale reference)")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured as one HIP graph and replayed")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the selection path is data-parallel over independent caches; see the "
              "sharding notes of the design)", file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2

    import torch
    from query_guided_kv_amd import kvsel as K
    from query_guided_kv_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a visible MI355X GPU", file=sys.stderr)
        return 2
    K.load()                                   # fails loudly if the library is missing
    dev = torch.device("cuda:0")

    if args.copy_probe:
        # a plain streaming kernel of known size: 1 GiB read, 1 GiB written
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
        log("copy probe: 3 x (1 GiB read + 1 GiB written) done")
    copy_GBps = device_copy_rate(dev)
    log(f"device copy: {copy_GBps:.0f} GB/s (read + written)")

    w = synth.workload(args.workload)
    res, inp, rows = measure(w, args.seed, args.steps, args.warmup, args.graph, copy_GBps, dev)
    result = dict({"metric": "cached KV tokens scored+selected per second",
                   "value": res["value"], "unit": "token-rows/s", "n_gpus": 1,
                   "steps": args.steps, "warmup": args.warmup,
                   "ms_per_step": res["ms_per_step"],
                   "ms_per_step_median": res["ms_per_step_median"],
                   "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
                   "dtype": w.dtype,
                   "data": "synthetic (seeded, planted relevant units; no datasets or weights)"},
                  **{k: v for k, v in res.items()
                     if k not in ("value", "ms_per_step", "ms_per_step_median", "dtype")})
    if not args.no_cpu:
        log("timing the CPU oracle on a sample")
        result["cpu_baseline"] = cpu_baselines(w, inp, w.recipe == "cachefocus")
    del inp
    if args.workload == DEFAULT_WORKLOAD and not args.no_also:
        torch.cuda.empty_cache()
        result["also"] = []
        for name, steps in ALSO:
            res_a, inp_a, _ = measure(synth.workload(name), args.seed, steps, 3, True, copy_GBps,
                                      dev)
            del inp_a
            torch.cuda.empty_cache()
            result["also"].append(also_entry(res_a))
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
