"""GPU parity of the index-based causal attention (kvsel_index_attn) against
the oracle's ``index_causal_attention``: outputs within 5e-3 absolute, lse
within 5e-3 (bf16 probabilities feed the value product, as in the MFMA decode).
"""

import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import announce, assert_rel, device
from oracle.pipeline import to64
from query_guided_kv_amd import kvsel as K
from query_guided_kv_amd import pipeline, synth

pytestmark = pytest.mark.gpu


def rnd(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (scale * torch.randn(shape, generator=g)).to(torch.bfloat16)


CASES = [
    # name, B, S, N, H, Hq, D, positions
    ("one_row_block_per_wave", 2, 37, 1000, 2, 8, 128, "sorted"),
    ("two_row_blocks_per_wave", 1, 1100, 3000, 2, 8, 128, "sorted"),
    ("d64_unsorted_edges", 2, 50, 700, 1, 4, 64, "edges"),
    ("gqa7_one_key_tiles", 1, 20, 130, 4, 28, 128, "sorted"),
    ("context_shorter_than_a_tile", 1, 9, 40, 2, 8, 64, "edges"),
]


def _positions(kind, B, S, N, rng):
    if kind == "sorted":
        return np.stack([np.sort(rng.choice(N, size=S, replace=False)) for _ in range(B)])
    p = rng.integers(0, N, size=(B, S))
    p[:, 0] = -1                   # attends to nothing
    p[:, 1] = 0                    # its own row only
    p[:, 2] = N + 50               # clipped to the last row
    p[:, 3] = N - 1
    return p


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_index_attn(case):
    name, B, S, N, H, Hq, D, kind = case
    announce("index_attn", case=name)
    dev = device()
    rng = np.random.default_rng(S + N)
    q = rnd((B, S, Hq, D), 1)
    k = rnd((B, N, H, D), 2, 1.5)
    v = rnd((B, N, H, D), 3)
    pos = _positions(kind, B, S, N, rng).astype(np.int32)
    o, lse = K.index_attn(q.to(dev), k.to(dev), v.to(dev), torch.from_numpy(pos).to(dev))
    torch.cuda.synchronize()
    wo, wl = O.index_causal_attention(to64(q), to64(k), to64(v), pos, 1 / np.sqrt(D))
    assert_rel(o, wo, 0.0, 5e-3, "output")
    fin = np.isfinite(wl)
    got_l = lse.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isfinite(got_l), fin)
    assert_rel(got_l[fin], wl[fin], 0.0, 5e-3, "lse")


def test_index_attn_special_cases():
    """Every position on the last row is the full attention of the decode call;
    every position 0 returns the first value row."""
    announce("index_attn_special")
    dev = device()
    B, S, N, H, Hq, D = 2, 40, 513, 2, 8, 128
    q, k, v = rnd((B, S, Hq, D), 4).to(dev), rnd((B, N, H, D), 5).to(dev), rnd((B, N, H, D), 6).to(dev)
    last = torch.full((B, S), N - 1, dtype=torch.int32, device=dev)
    o, lse = K.index_attn(q, k, v, last)
    od, lsed = K.decode_attn(q, [(k, v)])
    first = torch.zeros((B, S), dtype=torch.int32, device=dev)
    o0, _ = K.index_attn(q, k, v, first)
    torch.cuda.synchronize()
    assert_rel(o, to64(od), 0.0, 5e-3, "last position = full attention")
    assert_rel(lse, to64(lsed), 0.0, 5e-3, "lse")
    want0 = to64(v)[:, 0][:, None].repeat(S, axis=1).repeat(Hq // H, axis=2)
    np.testing.assert_allclose(to64(o0), want0, rtol=0, atol=1e-6)


def test_recompute_full_sampled_rows():
    """The 32-layer recomputation workload in the benchmark's configuration;
    sampled selected tokens of two layers against the oracle, every head."""
    w = synth.workload("infoflow_recompute_32l_64x1024")
    announce("recompute_full", workload=w.name)
    dev = device()
    inp = synth.generate(w, 0, dev)
    got = pipeline.RecomputePath(w, inp)(inp["q_sel"])
    torch.cuda.synchronize()
    S = inp["pos"].shape[1]
    pick = np.array([0, 1, 777, 4096, S // 2, S - 2, S - 1])
    for layer in (0, 29):
        q = to64(inp["q_sel"][layer:layer + 1])[:, pick]
        pos = inp["pos"][layer:layer + 1].cpu().numpy()[:, pick]
        wo, wl = O.index_causal_attention(q, to64(inp["k"][layer:layer + 1]),
                                          to64(inp["v"][layer:layer + 1]), pos, w.scale)
        assert_rel(got["o"][layer:layer + 1][:, pick], wo, 0.0, 5e-3, "output")
        assert_rel(got["lse"][layer:layer + 1][:, :, pick], wl, 0.0, 5e-3, "lse")
