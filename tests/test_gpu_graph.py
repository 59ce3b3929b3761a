"""Whole steps of the path captured in a HIP graph (torch.cuda.graph) and
replayed: every replay, with eager work and synchronisations between the
replays, must reproduce the eager step bit for bit.  Before each replay the
step's outputs are overwritten with a sentinel, so a replay that skipped a
write would show.  The library makes no memset, allocation or host
synchronisation inside a call, so a step is capturable as a whole.
"""

import pytest
import torch

from gpu_util import announce, device
from query_guided_kv_amd import pipeline, synth

pytestmark = pytest.mark.gpu

CASES = {
    # re-positioned scoring, chunk mass, aligned gather, decode
    "docs_small": lambda: synth.workload(
        "llama2_7b_32docs_x512", N=4096, Hq=8, H=8, T=8, k=4, window=1024,
        plants={"primary": 2, "primary_scale": 1.5, "secondary": 2, "secondary_scale": 1.25}),
    # token mass on the matrix cores (split over workgroup groups), refill, decode
    "bilayer_small": lambda: synth.workload(
        "acre_bilayer_l1_16k_l2_128k", N=2048, k=256,
        plants={"planted": 256, "gamma": 1.0, "l1_noise_std": 0.1}),
    # re-positioned keys kept, alpha * |v| over a layer group
    "infoflow_small": lambda: synth.workload(
        "infoflow_32l_64x1024", B=4, N=8192, group=4, k=1228,
        plants={"chunk_len": 1024, "chunks": 1, "chunk_scale": 1.5, "tokens": 204,
                "token_scale": 1.3}),
    # streaming scorer, fused refill + decode
    "serving_small": lambda: synth.workload(
        "serving_16req_8l_128k", B=4, requests=2, N=16384, k=8,
        plants={"chunks": 8, "gamma": 1.0, "query_topic": 2.0}),
}


def _tensors(inp: dict) -> list:
    return [t for t in inp.values() if isinstance(t, torch.Tensor)]


def _outputs(out: dict) -> dict:
    return {k: v for k, v in out.items() if isinstance(v, torch.Tensor)}


def _capture_and_check(step, inputs, replays: int = 3):
    eager = {k: v.clone() for k, v in _outputs(step()).items()}
    torch.cuda.synchronize()
    side = torch.cuda.Stream()          # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        got = _outputs(step())
    torch.cuda.synchronize()
    assert set(got) == set(eager)
    input_ptrs = {t.data_ptr() for t in inputs}
    for r in range(replays):
        for t in got.values():          # sentinel: a skipped write would show
            if t.data_ptr() not in input_ptrs:
                t.fill_(-3 if not t.is_floating_point() else -7.0)
        step()                          # eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, t in got.items():
            assert torch.equal(t, eager[k]), f"replay {r}: output {k} differs from the eager step"


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replay_path(name):
    w = CASES[name]()
    announce("graph_replay", case=name)
    dev = device()
    inp = synth.generate(w, 3, dev)
    path = pipeline.Path(w, inp)
    _capture_and_check(lambda: path(inp["q"]), _tensors(inp))


def test_graph_replay_prune_path():
    w = synth.workload("cachefocus_qwen2_28l_40docs_x512", requests=2, layers=6, prune_every=2,
                       N=8 * 128, unit_len=128, Hq=8, H=2, T=8, k=2, window=1 << 15)
    w = w.scaled(B=w.requests * w.layers)
    announce("graph_replay", case="prune")
    dev = device()
    inp = synth.generate(w, 7, dev)
    path = pipeline.PrunePath(w, inp)
    _capture_and_check(lambda: path(inp["q"], inp["q_dec"]), _tensors(inp))


def test_graph_replay_reorder_path():
    w = synth.workload("infoflow_reorder_32l_64x1024", B=4, N=8 * 256, group=4, k=612,
                       plants={"chunk_len": 256, "chunks": 2, "chunk_scale": 1.5,
                               "tokens": 100, "token_scale": 1.3})
    announce("graph_replay", case="reorder")
    dev = device()
    inp = synth.generate(w, 5, dev)
    path = pipeline.ReorderPath(w, inp)
    _capture_and_check(lambda: path(inp["q"]), _tensors(inp))


def test_graph_replay_recompute_path():
    w = synth.workload("infoflow_recompute_32l_64x1024", B=2, N=4096, group=2, k=600,
                       plants={"chunk_len": 1024, "chunks": 1, "chunk_scale": 1.5,
                               "tokens": 300, "token_scale": 1.3})
    announce("graph_replay", case="recompute")
    dev = device()
    inp = synth.generate(w, 6, dev)
    path = pipeline.RecomputePath(w, inp)
    _capture_and_check(lambda: path(inp["q_sel"]), _tensors(inp))
