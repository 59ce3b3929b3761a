"""Run-to-run reproducibility: the path has no floating-point atomics and
every reduction runs in a fixed order, so two runs on the same inputs give
the same bits.  Each workload runs twice through separate Path objects (their
own output buffers and workspaces), the second after the allocator's free
memory was filled with NaN, so a kernel that read memory it had not written
would show as a difference.
"""

import pytest
import torch

from gpu_util import announce, device
from query_guided_kv_amd import pipeline, synth

pytestmark = pytest.mark.gpu

CASES = {
    "docs_small": lambda: synth.workload(
        "llama2_7b_32docs_x512", N=4096, Hq=8, H=8, T=8, k=4, window=1024,
        plants={"primary": 2, "primary_scale": 1.5, "secondary": 2, "secondary_scale": 1.25}),
    "bilayer_small": lambda: synth.workload(
        "acre_bilayer_l1_16k_l2_128k", N=2048, k=256,
        plants={"planted": 256, "gamma": 1.0, "l1_noise_std": 0.1}),
    "infoflow_small": lambda: synth.workload(
        "infoflow_32l_64x1024", B=4, N=8192, group=4, k=1228,
        plants={"chunk_len": 1024, "chunks": 1, "chunk_scale": 1.5, "tokens": 204,
                "token_scale": 1.3}),
    "serving_small": lambda: synth.workload(
        "serving_16req_8l_128k", B=4, requests=2, N=16384, k=8,
        plants={"chunks": 8, "gamma": 1.0, "query_topic": 2.0}),
}


def _poison(dev, nbytes=1 << 30):
    """Fill 1 GiB of the caching allocator's memory with NaN and free it."""
    t = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    del t


@pytest.mark.parametrize("name", list(CASES))
def test_two_runs_give_the_same_bits(name):
    w = CASES[name]()
    announce("determinism", case=name)
    dev = device()
    inp = synth.generate(w, 4, dev)
    first = {k: v.clone() for k, v in pipeline.Path(w, inp)(inp["q"]).items()
             if isinstance(v, torch.Tensor)}
    torch.cuda.synchronize()
    _poison(dev)
    second = pipeline.Path(w, inp)(inp["q"])
    torch.cuda.synchronize()
    for key, t in first.items():
        assert torch.equal(t, second[key]), f"{name}: {key} differs between two runs"
