"""Refill from a host-resident L2 cache ([ACRE §2.2, §2.4]: L2 offloaded to CPU
memory, L1 kept on the GPU).

The gather kernels read the kept rows of pinned host tensors over the host
link.  Parity against the oracle is bit-exact for the copies (compact and
nested layouts) and within 5e-3 for the attention of kvsel_gather_decode.
Pageable host memory is refused before anything is launched.
"""

import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import announce, assert_rel, device
from oracle import pipeline as OP
from oracle.pipeline import to64
from query_guided_kv_amd import kvsel as K
from query_guided_kv_amd import pipeline, synth

pytestmark = pytest.mark.gpu


def rnd(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (scale * torch.randn(shape, generator=g)).to(torch.bfloat16)


def _idx(B, M, k, seed):
    rng = np.random.default_rng(seed)
    return np.stack([np.sort(rng.choice(M, size=k, replace=False)) for _ in range(B)])


@pytest.mark.parametrize("B,M,U,k,group", [(1, 2048, 8, 256, 1), (4, 300, 3, 77, 2)])
def test_gather_from_pinned_host(B, M, U, k, group):
    announce("gather_host", B=B, M=M, U=U, k=k, group=group)
    dev = device()
    H, D = 4, 128
    k2 = rnd((B, M * U, H, D), 1).pin_memory()
    v2 = rnd((B, M * U, H, D), 2).pin_memory()
    idx = _idx(B // group, M, k, 3)
    gk, gv = K.gather(k2, v2, torch.from_numpy(idx.astype(np.int32)).to(dev), U, group)
    torch.cuda.synchronize()
    assert gk.is_cuda and gv.is_cuda
    wk, wv = O.gather(to64(k2), to64(v2), np.repeat(idx, group, axis=0), U)
    np.testing.assert_array_equal(to64(gk), wk)
    np.testing.assert_array_equal(to64(gv), wv)


def test_nested_refill_from_pinned_host():
    announce("nested_host")
    dev = device()
    B, m, l, H, D, k = 2, 200, 8, 4, 128, 30
    l1k, l1v = rnd((B, m, H, D), 4).to(dev), rnd((B, m, H, D), 5).to(dev)
    l2k, l2v = rnd((B, m * l, H, D), 6).pin_memory(), rnd((B, m * l, H, D), 7).pin_memory()
    idx = _idx(B, m, k, 8)
    gk, gv = K.gather(l2k, l2v, torch.from_numpy(idx.astype(np.int32)).to(dev), l, 1,
                      proxy_k=l1k, proxy_v=l1v)
    torch.cuda.synchronize()
    for b in range(B):
        want_k = O.refill_nested(to64(l1k[b]), to64(l2k[b]), idx[b], l)
        want_v = O.refill_nested(to64(l1v[b]), to64(l2v[b]), idx[b], l)
        np.testing.assert_array_equal(to64(gk[b]), want_k)
        np.testing.assert_array_equal(to64(gv[b]), want_v)


@pytest.mark.parametrize("Hq,T", [(28, 1), (28, 16)])   # one-pass kernel; gather then decode
def test_gather_decode_from_pinned_host(Hq, T):
    announce("gather_decode_host", Hq=Hq, T=T)
    dev = device()
    B, M, U, k, H, D = 2, 512, 8, 64, 4, 128
    q = rnd((B, T, Hq, D), 9).to(dev)
    l1k, l1v = rnd((B, M, H, D), 10, 1.5).to(dev), rnd((B, M, H, D), 11).to(dev)
    l2k, l2v = rnd((B, M * U, H, D), 12, 1.5).pin_memory(), rnd((B, M * U, H, D), 13).pin_memory()
    idx = _idx(B, M, k, 14)
    gk, gv, o, lse = K.gather_decode(q, l2k, l2v, torch.from_numpy(idx.astype(np.int32)).to(dev),
                                     U, extra=[(l1k, l1v)])
    torch.cuda.synchronize()
    wk, wv = O.gather(to64(l2k), to64(l2v), idx, U)
    np.testing.assert_array_equal(to64(gk), wk)
    np.testing.assert_array_equal(to64(gv), wv)
    wo, wl = O.decode_attention(to64(q), [(to64(l1k), to64(l1v)), (wk, wv)], 1 / np.sqrt(D))
    assert_rel(o, wo, 0.0, 5e-3, "decode output")
    assert_rel(lse, wl, 0.0, 5e-3, "lse")


def test_pageable_host_memory_is_refused():
    # refused during validation: no kernel is launched, the output is untouched
    announce("pageable_refused")
    dev = device()
    k2 = rnd((1, 64, 4, 128), 15)                  # ordinary (pageable) host tensor
    assert not k2.is_pinned()
    idx = torch.tensor([[1, 5]], dtype=torch.int32, device=dev)
    with pytest.raises(K.KvselError) as e:
        K.gather(k2, None, idx, 4, 1)
    assert e.value.status == -4
    torch.cuda.synchronize()


def test_bilayer_path_with_host_l2():
    """The whole bi-layer path with L2 in pinned host memory, at full size,
    against the oracle (selection, refilled rows, decode)."""
    w = synth.workload("acre_bilayer_host_l2_l1_16k_l2_128k")
    announce("path_host_l2", workload=w.name)
    dev = device()
    inp = synth.generate(w, 0, dev)
    assert inp["l2_k"].is_pinned() and not inp["l2_k"].is_cuda
    got = pipeline.Path(w, inp)(inp["q"])
    torch.cuda.synchronize()
    want = OP.run(w, inp)
    idx = got["idx"].cpu().numpy().astype(np.int64)
    assert np.array_equal(idx, want["idx"]) and np.array_equal(idx[0], inp["planted"][0])
    np.testing.assert_array_equal(OP.to64(got["k_gather"]), want["k_gather"])
    np.testing.assert_array_equal(OP.to64(got["v_gather"]), want["v_gather"])
    assert_rel(got["o"], want["o"], 0.0, 5e-3, "decode output")
