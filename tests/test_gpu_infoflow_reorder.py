"""GPU parity of InfoFlow's two-stage selection with chunk reordering.

Per call: kvsel_unit_fractions and kvsel_slot_starts against the oracle,
bit-exact.  End to end: ReorderPath against the oracle's ``if_two_stage`` at
small sizes: both selections, the fractions, the order and the starts
bit-exact; scores within relative 2e-3; re-positioned keys within one bf16 ulp.
At the full 32-layer workload: the same exact relations between the GPU's own
intermediates, the plants, and the oracle on sampled layers.
"""

import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import announce, assert_cache_close, assert_rel, device
from oracle.pipeline import to64
from query_guided_kv_amd import kvsel as K
from query_guided_kv_amd import pipeline, synth

pytestmark = pytest.mark.gpu

MARGIN = 1e-2


@pytest.mark.parametrize("G,M,k,unit", [(1, 64, 9830, 1024), (3, 10, 37, 16), (2, 5, 0, 4),
                                        (4, 1, 3, 100)])
def test_unit_fractions(G, M, k, unit):
    announce("unit_fractions", G=G, M=M, k=k, unit=unit)
    dev = device()
    rng = np.random.default_rng(G * 7 + k)
    sel = np.stack([np.sort(rng.choice(M * unit, size=k, replace=False)) for _ in range(G)]) \
        if k else np.zeros((G, 0), np.int64)
    r = K.unit_fractions(torch.from_numpy(sel.astype(np.int32)).to(dev).contiguous(), unit, M)
    torch.cuda.synchronize()
    want = O.if_chunk_fractions(sel, [unit] * M)
    np.testing.assert_array_equal(np.rint(r.cpu().numpy().astype(np.float64) * unit),
                                  np.rint(want * unit))
    # equal counts give equal values, larger counts larger ones
    got = r.cpu().numpy()
    for g in range(G):
        a = np.argsort(want[g], kind="stable")
        assert np.all(np.diff(got[g][a]) >= 0)


@pytest.mark.parametrize("G,M,unit,rep", [(1, 64, 1024, 32), (3, 7, 96, 2), (2, 1, 5, 1)])
def test_slot_starts(G, M, unit, rep):
    announce("slot_starts", G=G, M=M, unit=unit, rep=rep)
    dev = device()
    rng = np.random.default_rng(M + rep)
    order = np.stack([rng.permutation(M) for _ in range(G)])
    delta = K.slot_starts(torch.from_numpy(order.astype(np.int32)).to(dev).contiguous(), unit,
                          rep=rep)
    torch.cuda.synchronize()
    want = np.repeat(O.if_reordered_offsets(order, [unit] * M), rep, axis=0)
    np.testing.assert_array_equal(delta.cpu().numpy(), want)


SMALL = {
    "mfma_two_chunks": dict(B=4, N=8 * 256, group=4, k=612,
                            plants={"chunk_len": 256, "chunks": 2, "chunk_scale": 1.5,
                                    "tokens": 100, "token_scale": 1.3}),
    # few query rows give noisy token scores: stronger plants keep the cuts
    # clear (oracle margins 18% and 12%)
    "two_requests_d64": dict(B=4, N=6 * 128, group=2, k=296, D=64, Hq=8, H=2, T=16,
                             plants={"chunk_len": 128, "chunks": 2, "chunk_scale": 2.0,
                                     "tokens": 40, "token_scale": 1.8}),
    "tile_fp32": dict(B=2, N=5 * 64, group=2, k=94, D=64, Hq=4, H=4, T=16, dtype="fp32",
                      plants={"chunk_len": 64, "chunks": 1, "chunk_scale": 2.2,
                              "tokens": 30, "token_scale": 2.0}),
}


def _margin(s, k):
    s = np.sort(np.asarray(s, np.float64))[::-1]
    return (s[k - 1] - s[k]) / s[k - 1]


@pytest.mark.parametrize("name", list(SMALL))
def test_reorder_path_small(name):
    w = synth.workload("infoflow_reorder_32l_64x1024", **SMALL[name])
    announce("reorder_path", case=name, B=w.B, N=w.N)
    dev = device()
    inp = synth.generate(w, 5, dev)
    got = pipeline.ReorderPath(w, inp)(inp["q"])
    torch.cuda.synchronize()
    lens = [int(w.plants["chunk_len"])] * (w.N // int(w.plants["chunk_len"]))
    want = O.if_two_stage(to64(inp["q"]), to64(inp["k"]), to64(inp["v"]), lens, w.scale, w.k,
                          w.group, w.rope_base, w.rope_style, w.dtype, w.signal)
    for g in range(w.B // w.group):
        assert _margin(want["score1"][g], w.k) > MARGIN and _margin(want["score2"][g], w.k) > MARGIN
    np.testing.assert_array_equal(got["sel1"].cpu().numpy(), want["sel1"])
    assert_rel(got["score1"], want["score1"], 2e-3, 0.0, "first-stage scores")
    np.testing.assert_array_equal(np.rint(got["r"].cpu().numpy().astype(np.float64) * lens[0]),
                                  np.rint(want["r"] * lens[0]))
    np.testing.assert_array_equal(got["order"].cpu().numpy(), want["order"])
    np.testing.assert_array_equal(got["delta"].cpu().numpy(),
                                  np.repeat(want["delta"], w.group, axis=0))
    assert_cache_close(got["k_rep"], want["k_rep"], w.dtype)
    np.testing.assert_array_equal(got["sel2"].cpu().numpy(), want["sel2"])
    assert_rel(got["score2"], want["score2"], 2e-3, 0.0, "second-stage scores")


def test_reorder_path_full_sampled_layers():
    """32 layers x 65,536 tokens, the benchmark's configuration.  Exact relations
    between the GPU's intermediates at full size, the plants, and the oracle on
    two sampled layers of the second stage (keys, row statistics, scores)."""
    w = synth.workload("infoflow_reorder_32l_64x1024")
    announce("reorder_full", workload=w.name)
    dev = device()
    inp = synth.generate(w, 0, dev)
    got = pipeline.ReorderPath(w, inp)(inp["q"])
    torch.cuda.synchronize()
    L = int(w.plants["chunk_len"])
    lens = [L] * (w.N // L)
    sel1 = got["sel1"].cpu().numpy().astype(np.int64)
    sel2 = got["sel2"].cpu().numpy().astype(np.int64)
    # both stages keep the planted tokens, by a margin
    assert np.array_equal(sel1[0], inp["planted"][0])
    assert np.array_equal(sel2[0], inp["planted"][0])
    for key, sel in (("score1", sel1), ("score2", sel2)):
        s = got[key].cpu().numpy()[0].astype(np.float64)
        kept = np.zeros(w.N, bool)
        kept[sel[0]] = True
        assert s[kept].min() > s[~kept].max() * (1 + MARGIN), key
    # fractions, order and starts follow from the first selection exactly
    r = O.if_chunk_fractions(sel1, lens)
    np.testing.assert_array_equal(np.rint(got["r"].cpu().numpy().astype(np.float64) * L),
                                  np.rint(r * L))
    order = O.if_reorder(r)
    np.testing.assert_array_equal(got["order"].cpu().numpy(), order)
    assert set(order[0, -6:].tolist()) == set(inp["planted_chunks"].tolist())
    delta = O.if_reordered_offsets(order, lens)
    np.testing.assert_array_equal(got["delta"].cpu().numpy(), np.repeat(delta, w.B, axis=0))
    # two sampled layers of the second stage against the oracle, in full
    rm, rs, _ = K.score(inp["q"], got["k_rep"], 1, w.scale, row_stats=True, partials=False)
    per_layer = K.aggregate(1, 1, "vnorm", q=inp["q"], k=got["k_rep"], v=inp["v"],
                            row_max=rm, row_sum=rs, scale=w.scale)
    torch.cuda.synchronize()
    assert_rel(per_layer.double().sum(0, keepdim=True).cpu().numpy(),
               got["score2"].cpu().numpy().astype(np.float64), 1e-4, 0.0, "sum over layers")
    local = np.tile(np.arange(L), len(lens))
    p_new = local + np.repeat(delta[0], L)
    for layer in (0, 19):
        k64 = to64(inp["k"][layer:layer + 1])
        k2 = O.reposition(k64, local[None], p_new[None], w.rope_base, w.rope_style, w.dtype)
        assert_cache_close(got["k_rep"][layer:layer + 1], k2, w.dtype)
        m, Z, _ = O.score(to64(inp["q"][layer:layer + 1]), k2, w.scale, 1)
        assert_rel(rm[layer:layer + 1], m, 2e-3, 2e-3, "row_max")
        assert_rel(rs[layer:layer + 1], Z, 2e-3, 0.0, "row_sum")
        s = O.aggregate(to64(inp["q"][layer:layer + 1]), k2, to64(inp["v"][layer:layer + 1]),
                        w.scale, "vnorm", 1, 1)
        assert_rel(per_layer[layer:layer + 1], s, 2e-3, 0.0, "layer scores")
