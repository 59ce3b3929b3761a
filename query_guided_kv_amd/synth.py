"""Seeded synthetic inputs for query-guided KV selection.

This module draws random caches and query blocks with the shapes of the
workloads described on the source pages, and plants relevant units so that the
selected set is decided by a wide margin rather than by rounding noise.  It
holds none of the selection method's arithmetic: no rotation, no softmax, no
ranking.  Both the HIP path and the CPU oracle read the same tensors from here.

Host workloads are drawn with numpy's PCG64; the two large ones are drawn with
torch's generator on whatever device is given (Philox on a GPU), so that tens
of GB never cross the host link.

Plants (a "unit" is a chunk, document, L1 entry or token that is scored):

* key scaling: multiplying a unit's keys by ``s`` raises the expected
  ``exp(q.k / sqrt(D))`` over isotropic queries from ``e^(1/2)`` to
  ``e^(s^2/2)``.  A rotation keeps the norm, so the plant survives any
  re-positioning of the keys (used where keys are re-rotated);
* query-aligned offset: adding ``gamma * sqrt(D) * qbar / |qbar|^2`` to a key
  raises the mean logit of the rows averaged in ``qbar`` by exactly ``gamma``
  (used where keys are scored in the frame they are stored in);
* topic vectors: a unit vector ``u`` is added to the keys of the planted chunks
  (times ``gamma * sqrt(D)``) and to every query (times 2).
"""

from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "workload", "generate", "serving_queries"]


@dataclass(frozen=True)
class Workload:
    """Shape of one workload.  Caches are ``[B][N][H][D]``, queries ``[B][T][Hq][D]``."""

    name: str
    recipe: str          # generator: "tiny", "docs", "bilayer", "infoflow", "serving",
                         # "cachefocus"
    B: int               # independent instances (requests x layers, or layers)
    N: int               # cached rows scored per instance
    Hq: int              # query heads
    H: int               # kv heads
    D: int               # head dim
    T: int               # query tokens
    dtype: str           # "bf16" or "fp32"
    unit_len: int        # rows per scored unit (chunk / document; 1 = token)
    k: int               # units kept per selection group
    group: int = 1       # consecutive instances whose scores are summed
    signal: str = "mass"          # "mass" or "vnorm"
    reposition: str = "none"      # "none", "contiguous", "reuse_window", "global"
    window: int = 0               # positional window (reuse_window)
    align: bool = False           # re-position the kept units to contiguous slots
    refill_interval: int = 0      # L2 rows per L1 entry (bi-layer refill)
    decode: bool = True           # run the final attention pass
    rope_base: float = 10000.0
    rope_style: str = "half"
    plants: Dict[str, float] = field(default_factory=dict)
    steps: int = 1                # decode steps with fresh queries (serving)
    requests: int = 1             # serving: requests (B = requests * layers)
    layers: int = 1               # layer-wise pruning: layers per request
    prune_every: int = 0          # layer-wise pruning: prune after every n-th layer
    allocation: str = "align"     # layer-wise pruning: final order, "align" or "sort"
    reorder: bool = False         # two-stage selection with chunk reordering
    l2_host: bool = False         # bi-layer refill: L2 cache in pinned host memory
    recompute: bool = False       # attention of the selected tokens to the context

    @property
    def M(self) -> int:
        return self.N // self.unit_len

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.D))

    def scaled(self, **over) -> "Workload":
        """A copy with some fields replaced (smaller test sizes)."""
        return dataclasses.replace(self, **over)


WORKLOADS: Dict[str, Workload] = {
    # 1 layer, 4-head MHA, head dim 64, fp32; 8 chunks x 128 cached tokens; a
    # 16-token query; chunks 3 and 6 get +0.5 * mean(query) added to their keys;
    # chunks re-positioned to contiguous positions; keep 2 chunks by summed
    # attention mass; gather; decode.
    "tiny_mha4_d64_fp32_8x128": Workload(
        name="tiny_mha4_d64_fp32_8x128", recipe="tiny", B=1, N=1024, Hq=4, H=4, D=64, T=16,
        dtype="fp32", unit_len=128, k=2, reposition="contiguous",
        plants={"mean_query": 0.5}),
    # LLaMA-2-7B-shaped layer: 32-head MHA, head dim 128, bf16; 32 documents x
    # 512 tokens at local positions; 32-token query; documents re-positioned
    # into a 4096-position window; keep 8 by attention mass; gather with the
    # kept documents re-positioned to contiguous slots; decode.
    "llama2_7b_32docs_x512": Workload(
        name="llama2_7b_32docs_x512", recipe="docs", B=1, N=16384, Hq=32, H=32, D=128, T=32,
        dtype="bf16", unit_len=512, k=8, reposition="reuse_window", window=4096,
        align=True, plants={"primary": 4, "primary_scale": 1.5,
                            "secondary": 4, "secondary_scale": 1.25}),
    # Bi-layer refill: GQA 28/4, head dim 128, bf16; L2 cache 131072 rows, L1
    # cache 16384 entries (one per 8 L2 rows: mean of the 8 plus N(0, 0.1^2));
    # a 64-token query attends L1; the top 2048 entries are refilled with their
    # 8 L2 rows each; decode over L1 plus the refilled rows.
    "acre_bilayer_l1_16k_l2_128k": Workload(
        name="acre_bilayer_l1_16k_l2_128k", recipe="bilayer", B=1, N=16384, Hq=28, H=4, D=128, T=64,
        dtype="bf16", unit_len=1, k=2048, refill_interval=8,
        plants={"planted": 2048, "gamma": 1.0, "l1_noise_std": 0.1}),
    # The same bi-layer cache with L2 offloaded to (pinned) host memory and L1
    # kept on the GPU: the refill reads only the kept L2 blocks over the host
    # link.
    "acre_bilayer_host_l2_l1_16k_l2_128k": Workload(
        name="acre_bilayer_host_l2_l1_16k_l2_128k", recipe="bilayer", B=1, N=16384, Hq=28,
        H=4, D=128, T=64, dtype="bf16", unit_len=1, k=2048, refill_interval=8, l2_host=True,
        plants={"planted": 2048, "gamma": 1.0, "l1_noise_std": 0.1}),
    # Token-level recompute selection: 32 layers, GQA 32/8, head dim 128, bf16;
    # 64 chunks x 1024 tokens at chunk-local positions; re-rotated to global
    # positions; per-token score = sum over heads, 32 query tokens and layers of
    # attention weight x ||v||_2; keep the top 15% of tokens (indices only).
    "infoflow_32l_64x1024": Workload(
        name="infoflow_32l_64x1024", recipe="infoflow", B=32, N=65536, Hq=32, H=8, D=128, T=32,
        dtype="bf16", unit_len=1, k=9830, group=32, signal="vnorm",
        reposition="global", decode=False,
        plants={"chunk_len": 1024, "chunks": 6, "chunk_scale": 1.5,
                "tokens": 3686, "token_scale": 1.3}),
    # The same caches with chunk reordering: a first selection on the stored
    # chunk-local keys (the prompt at its global position), the share r_i of
    # each chunk's tokens in it, the chunks reordered with the most informative
    # nearest the prompt, GLOBAL positions rebuilt for that order, and the
    # same 15% budget selected again.
    "infoflow_reorder_32l_64x1024": Workload(
        name="infoflow_reorder_32l_64x1024", recipe="infoflow", B=32, N=65536, Hq=32, H=8,
        D=128, T=32, dtype="bf16", unit_len=1, k=9830, group=32, signal="vnorm",
        reposition="global", decode=False, reorder=True,
        plants={"chunk_len": 1024, "chunks": 6, "chunk_scale": 1.5,
                "tokens": 3686, "token_scale": 1.3}),
    # Recomputation of the selected tokens on the same caches: the 9830 selected
    # tokens (the planted 15%) of every layer attend causally to the context
    # up to their own positions, with fresh queries.
    "infoflow_recompute_32l_64x1024": Workload(
        name="infoflow_recompute_32l_64x1024", recipe="infoflow", B=32, N=65536, Hq=32, H=8,
        D=128, T=32, dtype="bf16", unit_len=1, k=9830, group=32, signal="vnorm",
        reposition="global", decode=False, recompute=True,
        plants={"chunk_len": 1024, "chunks": 6, "chunk_scale": 1.5,
                "tokens": 3686, "token_scale": 1.3}),
    # Batched serving: 16 requests x 8 layers, 131072 cached tokens each, GQA
    # 32/8, head dim 128, bf16 (~68.7 GB of K and V); per decode step a 1-token
    # query per (request, layer) scores the whole cache, keeps 64 chunks of 256
    # tokens, gathers them and runs decode attention; 128 steps.
    "serving_16req_8l_128k": Workload(
        name="serving_16req_8l_128k", recipe="serving", B=128, N=131072, Hq=32, H=8, D=128, T=1,
        dtype="bf16", unit_len=256, k=64, requests=16, steps=128,
        plants={"chunks": 64, "gamma": 1.0, "query_topic": 2.0}),
    # Layer-adaptive cache pruning on a Qwen2-7B-shaped model: 28 layers, GQA
    # 28/4, head dim 128, bf16, a 32K positional range.  Per request, 40
    # retrieved documents x 512 tokens are cached per layer at document-local
    # positions and a 32-token query block arrives per layer.  Every layer
    # re-positions the current documents to consecutive slots, scores them and
    # accumulates document-wise attention; every 4th layer prunes 5 (40 -> 5
    # over 7 pruning layers).  The 5 survivors are re-positioned to consecutive
    # slots in order of relevance ("sort") for all 28 layers, and one decode
    # step (1 query token per layer) attends them.  16 requests (B = 16 x 28
    # caches); document relevance planted as a ramp of key scales.
    "cachefocus_qwen2_28l_40docs_x512": Workload(
        name="cachefocus_qwen2_28l_40docs_x512", recipe="cachefocus", B=16 * 28, N=40 * 512,
        Hq=28, H=4, D=128, T=32, dtype="bf16", unit_len=512, k=5, reposition="reuse_window",
        window=32768, requests=16, layers=28, prune_every=4, allocation="sort",
        plants={"top_scale": 1.6, "scale_step": 0.025}),
}


def workload(name: str, **over) -> Workload:
    w = WORKLOADS[name]
    return w.scaled(**over) if over else w


# ---------------------------------------------------------------------------
# helpers (no method arithmetic)
# ---------------------------------------------------------------------------

_TORCH_DTYPE = {"bf16": torch.bfloat16, "fp32": torch.float32}


def _to_cache(x: np.ndarray, dtype: str, device) -> torch.Tensor:
    """float32 numpy -> torch tensor of the cache dtype (round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(_TORCH_DTYPE[dtype]).to(device)


def _query_aligned(qbar: np.ndarray, gamma: float) -> np.ndarray:
    """Offset that raises the mean logit (scale 1/sqrt(D)) of the averaged rows by gamma."""
    D = qbar.shape[-1]
    return gamma * np.sqrt(D) * qbar / np.sum(qbar * qbar, axis=-1, keepdims=True)


# ---------------------------------------------------------------------------
# generators
# ---------------------------------------------------------------------------

def generate(w: Workload, seed: int = 0, device="cpu") -> dict:
    """Draw one input batch of workload ``w``.

    Returns a dict with ``q``, ``k``, ``v`` (torch tensors on ``device``), the
    ``planted`` unit indices per selection group (a list of sorted int arrays;
    these fill exactly ``k`` slots), and workload specific extras (``l1_k``,
    ``l1_v`` for the bi-layer cache).  Keys are stored at unit-local positions
    when the workload re-positions them.
    """
    gen = {"tiny": _gen_tiny, "docs": _gen_docs, "bilayer": _gen_bilayer,
           "infoflow": _gen_infoflow, "serving": _gen_serving,
           "cachefocus": _gen_cachefocus}[w.recipe]
    return gen(w, seed, device)


def _gen_tiny(w: Workload, seed: int, device) -> dict:
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((w.B, w.T, w.Hq, w.D), dtype=np.float32)
    k = rng.standard_normal((w.B, w.N, w.H, w.D), dtype=np.float32)
    v = rng.standard_normal((w.B, w.N, w.H, w.D), dtype=np.float32)
    planted = sorted(u for u in (3, 6) if u < w.M)
    # per-head mean over the query tokens (kv head g takes the mean of its group)
    qbar = q.reshape(w.B, w.T, w.H, w.Hq // w.H, w.D).mean(axis=(1, 3))   # [B][H][D]
    for u in planted:
        k[:, u * w.unit_len:(u + 1) * w.unit_len] += w.plants["mean_query"] * qbar[:, None]
    return dict(q=_to_cache(q, w.dtype, device), k=_to_cache(k, w.dtype, device),
                v=_to_cache(v, w.dtype, device),
                planted=[np.array(planted, dtype=np.int64)] * (w.B // w.group))


def _gen_docs(w: Workload, seed: int, device) -> dict:
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((w.B, w.T, w.Hq, w.D), dtype=np.float32)
    k = rng.standard_normal((w.B, w.N, w.H, w.D), dtype=np.float32)
    v = rng.standard_normal((w.B, w.N, w.H, w.D), dtype=np.float32)
    n1, n2 = int(w.plants["primary"]), int(w.plants["secondary"])
    chosen = rng.choice(w.M, size=n1 + n2, replace=False)
    U = w.unit_len
    for i, u in enumerate(chosen):
        s = w.plants["primary_scale"] if i < n1 else w.plants["secondary_scale"]
        k[:, u * U:(u + 1) * U] *= np.float32(s)
    return dict(q=_to_cache(q, w.dtype, device), k=_to_cache(k, w.dtype, device),
                v=_to_cache(v, w.dtype, device),
                planted=[np.sort(chosen).astype(np.int64)] * (w.B // w.group),
                primary=np.sort(chosen[:n1]).astype(np.int64))


def _gen_bilayer(w: Workload, seed: int, device) -> dict:
    """L2 rows ~ N(0,1); L1 entry j = mean of L2 rows [l*j, l*(j+1)) + N(0, std^2)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    l = w.refill_interval
    n2 = w.N * l
    q = rng.standard_normal((w.B, w.T, w.Hq, w.D), dtype=np.float32)
    k2 = rng.standard_normal((w.B, n2, w.H, w.D), dtype=np.float32)
    v2 = rng.standard_normal((w.B, n2, w.H, w.D), dtype=np.float32)
    n_plant = int(w.plants["planted"])
    chosen = np.sort(rng.choice(w.N, size=n_plant, replace=False))
    # qbar per kv head: mean over the group's query heads and tokens
    qbar = q.reshape(w.B, w.T, w.H, w.Hq // w.H, w.D).mean(axis=(1, 3))     # [B][H][D]
    off = _query_aligned(qbar, w.plants["gamma"]).astype(np.float32)        # [B][H][D]
    k2r = k2.reshape(w.B, w.N, l, w.H, w.D)
    k2r[:, chosen] += off[:, None, None]
    # round L2 first: the L1 entries summarise the stored L2 rows
    k2t = _to_cache(k2, w.dtype, "cpu")
    v2t = _to_cache(v2, w.dtype, "cpu")
    std = w.plants["l1_noise_std"]
    k1 = k2t.float().numpy().reshape(w.B, w.N, l, w.H, w.D).mean(axis=2)
    v1 = v2t.float().numpy().reshape(w.B, w.N, l, w.H, w.D).mean(axis=2)
    k1 = k1 + std * rng.standard_normal(k1.shape, dtype=np.float32)
    v1 = v1 + std * rng.standard_normal(v1.shape, dtype=np.float32)
    if w.l2_host:   # a fresh pinned (page-locked) host allocation the GPU can read
        l2_k, l2_v = k2t.pin_memory(), v2t.pin_memory()
    else:
        l2_k, l2_v = k2t.to(device), v2t.to(device)
    return dict(q=_to_cache(q, w.dtype, device),
                k=_to_cache(k1, w.dtype, device), v=_to_cache(v1, w.dtype, device),
                l2_k=l2_k, l2_v=l2_v,
                planted=[chosen.astype(np.int64)] * (w.B // w.group))


def _device_generator(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _gen_infoflow(w: Workload, seed: int, device) -> dict:
    """Per-layer caches at chunk-local positions; planted chunks and tokens are
    shared by all layers (one selection for all layers)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    g = _device_generator(seed, device)
    td = _TORCH_DTYPE[w.dtype]
    q = torch.empty((w.B, w.T, w.Hq, w.D), dtype=td, device=device)
    k = torch.empty((w.B, w.N, w.H, w.D), dtype=td, device=device)
    v = torch.empty((w.B, w.N, w.H, w.D), dtype=td, device=device)
    q.normal_(generator=g)
    for b in range(w.B):
        k[b].normal_(generator=g)
        v[b].normal_(generator=g)
    C = int(w.plants["chunk_len"])
    n_chunks = w.N // C
    chunks = np.sort(rng.choice(n_chunks, size=int(w.plants["chunks"]), replace=False))
    in_chunk = np.zeros(w.N, dtype=bool)
    for c in chunks:
        in_chunk[c * C:(c + 1) * C] = True
    free = np.flatnonzero(~in_chunk)
    tokens = np.sort(rng.choice(free, size=int(w.plants["tokens"]), replace=False))
    scale = torch.ones(w.N, dtype=torch.float32)
    scale[torch.from_numpy(np.flatnonzero(in_chunk))] = float(w.plants["chunk_scale"])
    scale[torch.from_numpy(tokens)] = float(w.plants["token_scale"])
    scale = scale.to(device)[:, None, None]
    for b in range(w.B):
        k[b] = (k[b].float() * scale).to(td)
    planted = np.sort(np.concatenate([np.flatnonzero(in_chunk), tokens])).astype(np.int64)
    out = dict(q=q, k=k, v=v, planted=[planted] * (w.B // w.group),
               planted_chunks=chunks.astype(np.int64), planted_tokens=tokens)
    if w.recompute:
        # queries of the selected tokens, one block per layer, and their positions
        S = planted.size
        qs = torch.empty((w.B, S, w.Hq, w.D), dtype=td, device=device)
        qs.normal_(generator=g)
        out["q_sel"] = qs
        out["pos"] = torch.from_numpy(np.tile(planted.astype(np.int32), (w.B, 1))).to(device)
    return out


def _gen_serving(w: Workload, seed: int, device) -> dict:
    """Per (request, kv head) a unit topic vector u; per (request, layer) instance
    ``chunks`` random chunks get ``gamma*sqrt(D)*u`` added to every key.  Queries
    for each step are drawn by :func:`serving_queries`."""
    rng = np.random.Generator(np.random.PCG64(seed))
    g = _device_generator(seed, device)
    td = _TORCH_DTYPE[w.dtype]
    layers = w.B // w.requests
    topic = rng.standard_normal((w.requests, w.H, w.D))
    topic /= np.linalg.norm(topic, axis=-1, keepdims=True)
    k = torch.empty((w.B, w.N, w.H, w.D), dtype=td, device=device)
    v = torch.empty((w.B, w.N, w.H, w.D), dtype=td, device=device)
    planted = []
    U = w.unit_len
    amp = float(w.plants["gamma"]) * float(np.sqrt(w.D))
    for b in range(w.B):
        k[b].normal_(generator=g)
        v[b].normal_(generator=g)
        ch = np.sort(rng.choice(w.M, size=int(w.plants["chunks"]), replace=False))
        planted.append(ch.astype(np.int64))
        off = torch.from_numpy((amp * topic[b // layers]).astype(np.float32)).to(device)
        idx = torch.from_numpy(ch).to(device)
        kb = k[b].view(w.M, U, w.H, w.D)
        kb[idx] = (kb[idx].float() + off).to(td)
    return dict(k=k, v=v, topic=topic.astype(np.float32), planted=planted,
                q=serving_queries(w, topic, seed, 0, device))


def serving_queries(w: Workload, topic: np.ndarray, seed: int, step: int, device) -> torch.Tensor:
    """Fresh query block for one decode step: ``q = z + 2*u`` per (request, head)."""
    g = _device_generator(seed * 100003 + 7919 * (step + 1), device)
    td = _TORCH_DTYPE[w.dtype]
    layers = w.B // w.requests
    z = torch.empty((w.B, w.T, w.Hq, w.D), dtype=torch.float32, device=device)
    z.normal_(generator=g)
    per_head = np.repeat(np.asarray(topic, np.float32), w.Hq // w.H, axis=1)   # [R][Hq][D]
    per_inst = np.repeat(per_head, layers, axis=0)                              # [B][Hq][D]
    u = torch.from_numpy(per_inst).to(device)[:, None]
    return (z + float(w.plants["query_topic"]) * u).to(td)


def _gen_cachefocus(w: Workload, seed: int, device) -> dict:
    """Per request a random relevance rank of its documents (0 = most
    relevant); the keys of the document of rank r are scaled by
    ``top_scale - scale_step * r`` at every layer (raising its expected
    ``exp`` logit against isotropic queries to ``e^(s^2/2)``; a rotation keeps
    the scale).  Caches are ``[requests * layers][N][H][D]``, request-major;
    pre-fill query blocks ``q`` are ``[layers][requests][T][Hq][D]`` (one block
    per layer and request); ``q_dec`` holds one decode token per cache,
    ``[requests * layers][1][Hq][D]``.  ``planted`` lists each request's
    ``k`` documents of best rank."""
    rng = np.random.Generator(np.random.PCG64(seed))
    g = _device_generator(seed, device)
    td = _TORCH_DTYPE[w.dtype]
    R, L, U = w.requests, w.layers, w.unit_len
    if w.B != R * L:
        raise ValueError("cachefocus workloads need B = requests * layers")
    n_docs = w.M
    q = torch.empty((L, R, w.T, w.Hq, w.D), dtype=td, device=device)
    q.normal_(generator=g)
    q_dec = torch.empty((w.B, 1, w.Hq, w.D), dtype=td, device=device)
    q_dec.normal_(generator=g)
    rank = np.stack([rng.permutation(n_docs) for _ in range(R)])
    scale = (w.plants["top_scale"] - w.plants["scale_step"] * rank).astype(np.float32)
    k = torch.empty((w.B, w.N, w.H, w.D), dtype=td, device=device)
    v = torch.empty((w.B, w.N, w.H, w.D), dtype=td, device=device)
    for b in range(w.B):
        k[b].normal_(generator=g)
        v[b].normal_(generator=g)
        s = torch.from_numpy(scale[b // L]).to(device)[:, None, None, None]
        k[b] = (k[b].float().view(n_docs, U, w.H, w.D) * s).view(w.N, w.H, w.D).to(td)
    planted = [np.sort(np.flatnonzero(rank[r] < w.k)).astype(np.int64) for r in range(R)]
    return dict(q=q, q_dec=q_dec, k=k, v=v, planted=planted, rank=rank)
