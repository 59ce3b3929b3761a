"""kvsel_gather_decode_noalloc against kvsel_gather_decode.

The no-allocation variant keeps the split partials in the library's fixed
device array instead of a caller workspace; everything else is the same call.
On the GPU, two calls in a row (the second smaller, so the array holds the
first call's partials when the second starts) of each decode path -- the
one-pass streaming refill + decode and the copy followed by the matrix-core
pass with an extra segment -- are compared with the workspace entry point:
compact caches bit-exact, outputs within 5e-3 and log-sum-exp within 2e-3
absolute.  On the CPU, a shape whose partials exceed the array is refused
before anything is enqueued.
"""

import ctypes

import pytest
import torch

from query_guided_kv_amd import abi
from query_guided_kv_amd import kvsel as K


def _inputs(B, N, H, D, Hq, T, unit, kept, seed, extra_rows=0):
    g = torch.Generator().manual_seed(seed)
    dev = torch.device("cuda:0")
    k = torch.randn((B, N, H, D), generator=g).to(torch.bfloat16).to(dev)
    v = torch.randn((B, N, H, D), generator=g).to(torch.bfloat16).to(dev)
    q = torch.randn((B, T, Hq, D), generator=g).to(torch.bfloat16).to(dev)
    M = N // unit
    idx = torch.stack([torch.sort(torch.randperm(M, generator=g)[:kept]).values
                       for _ in range(B)]).to(torch.int32).to(dev)
    extra = []
    if extra_rows:
        ek = torch.randn((B, extra_rows, H, D), generator=g).to(torch.bfloat16).to(dev)
        ev = torch.randn((B, extra_rows, H, D), generator=g).to(torch.bfloat16).to(dev)
        extra = [(ek, ev)]
    return q, k, v, idx, extra


CASES = {
    # one-pass streaming refill + decode (4 query rows per kv head): 65 MiB of
    # partials at 16 requests x 8 layers; here two smaller shapes in a row
    "stream": [dict(B=16, N=32768, H=8, D=128, Hq=32, T=1, unit=256, kept=32, seed=1),
               dict(B=4, N=8192, H=8, D=128, Hq=32, T=1, unit=256, kept=8, seed=2)],
    # copy, then the matrix-core pass over an extra segment plus the copy
    "mfma_extra": [dict(B=2, N=16384, H=4, D=128, Hq=28, T=4, unit=8, kept=1024, seed=3,
                        extra_rows=4096),
                   dict(B=1, N=4096, H=4, D=128, Hq=28, T=4, unit=8, kept=128, seed=4,
                        extra_rows=1024)],
}


@pytest.mark.gpu
@pytest.mark.parametrize("case", list(CASES))
def test_noalloc_matches_workspace_call(case):
    print(f"[gpu-case] gather_decode_noalloc case={case}", flush=True)
    assert torch.cuda.is_available()
    for call, shape in enumerate(CASES[case]):
        q, k, v, idx, extra = _inputs(**shape)
        unit = shape["unit"]
        kd, vd, o, lse = K.gather_decode(q, k, v, idx, unit, extra=extra)
        kd2, vd2, o2, lse2 = K.gather_decode_noalloc(q, k, v, idx, unit, extra=extra)
        torch.cuda.synchronize()
        assert torch.equal(kd, kd2), f"call {call}: compact keys"
        assert torch.equal(vd, vd2), f"call {call}: compact values"
        assert (o - o2).abs().max().item() <= 5e-3, f"call {call}: decode output"
        assert (lse - lse2).abs().max().item() <= 2e-3, f"call {call}: lse"


def test_noalloc_refuses_shapes_beyond_the_array():
    # CPU only: the size check runs before anything touches a device
    lib = abi.load()
    cap = lib.kvsel_noalloc_scratch_bytes()
    assert cap == 128 << 20
    B, N, H, D, Hq, T, unit, kept = 1024, 131072, 8, 128, 32, 1, 256, 64
    kc = abi.Cache(B, N, H, D, N * H * D, H * D, abi.BF16)
    need = lib.kvsel_gather_decode_workspace(T, Hq, kc, unit, kept, None, 0)
    assert need > cap
    p = ctypes.c_void_p(0x10000)
    rc = lib.kvsel_gather_decode_noalloc(p, T, Hq, 0.088, p, p, kc, unit, p, kept, 1, p, p, None,
                                         0, p, None, None)
    assert rc == abi.ERR_WORKSPACE
    assert b"scratch" in lib.kvsel_last_error()
    # the serving shape (16 requests x 8 layers, 64 chunks of 256 kept) fits
    kc = abi.Cache(128, N, H, D, N * H * D, H * D, abi.BF16)
    assert lib.kvsel_gather_decode_workspace(T, Hq, kc, unit, kept, None, 0) <= cap
