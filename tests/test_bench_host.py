"""Host logic of bench.py, no GPU: every kernel a bench line can name for a
stage of any workload has its sources listed (for the stored-traffic hash)
and is a kernel of the built library; every stage is counted either as
selection or as refill / attention."""

import pytest
import torch

import bench
from query_guided_kv_amd import kvsel, pipeline, synth

OTHER_STAGES = {"gather", "decode", "gather_decode", "final_gather", "recompute"}


def stages_of(w):
    if w.recipe == "cachefocus":
        return pipeline.PrunePath.STAGES
    if w.recompute:
        return pipeline.RecomputePath.STAGES
    small = w.scaled(B=max(w.group, 1), requests=1)
    dummy = {"k": torch.zeros(1), "v": torch.zeros(1), "q": torch.zeros(1)}
    return pipeline.make_path(small, dummy).stages


@pytest.mark.parametrize("name", sorted(synth.WORKLOADS))
def test_stage_kernels_are_known(name):
    w = synth.workload(name)
    with open(kvsel.LIB_PATH, "rb") as f:
        lib = f.read()
    for stage in stages_of(w):
        kernel = bench.kernel_of(stage, w)
        for k in kernel.split("+"):
            assert k in bench.KERNEL_SOURCES, (stage, k)
            assert k.encode() in lib, f"{k} is not a kernel of {kvsel.LIB_PATH}"
        assert len(bench.source_hash(kernel)) == 16
        assert stage in bench.SELECTION_STAGES or stage in OTHER_STAGES, stage


def test_topk_kernel_follows_row_length():
    serving = synth.workload("serving_16req_8l_128k")        # 512 units per row
    infoflow = synth.workload("infoflow_32l_64x1024")        # 65,536 tokens per row
    longer = synth.workload("infoflow_32l_64x1024", N=131072)
    assert bench.kernel_of("topk", serving) == "topk_reg_kernel"
    assert bench.kernel_of("topk", infoflow) == "topk_reg_kernel"   # 64 keys per thread
    assert bench.kernel_of("topk", longer) == "topk_stream_kernel"


def test_host_cpu_record():
    h = bench.host_cpu()
    assert h["cpu_count"] >= 1 and 1 <= h["affinity"] <= h["cpu_count"]
