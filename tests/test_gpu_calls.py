"""GPU parity of each library call against the oracle, element by element.

Sizes are small enough for the oracle to finish in seconds but span several
workgroup tiles, splits and segments, with ragged tails, and cover every
kernel path (stream / tile, bf16 / fp32, head dim 64 / 128, both RoPE
pairings).  Tolerances: re-rotated keys within one bf16 ulp (>= 99.9% equal),
scores within relative 2e-3, decode outputs within 5e-3 absolute, indices and
copies bit-exact.
"""

import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import announce, assert_cache_close, assert_rel, device
from oracle.pipeline import to64
from query_guided_kv_amd import kvsel as K

pytestmark = pytest.mark.gpu

TD = {"bf16": torch.bfloat16, "fp32": torch.float32}
STYLE = {"half": "half", "interleaved": "interleaved"}


def rnd(shape, dtype, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (scale * torch.randn(shape, generator=g)).to(TD[dtype])


# --------------------------------------------------------------------------
# kvsel_reposition
# --------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,D,style,unit,N,per_inst", [
    ("bf16", 128, "half", 40, 1000, False),
    ("bf16", 128, "interleaved", 8, 520, True),
    ("bf16", 64, "half", 1, 77, True),
    ("fp32", 64, "half", 128, 1024, False),
    ("fp32", 128, "interleaved", 5, 335, True),
])
def test_reposition(dtype, D, style, unit, N, per_inst):
    announce("reposition", dtype=dtype, D=D, style=style, unit=unit, N=N, per_inst=per_inst)
    dev = device()
    B, H = 3, 4
    k = rnd((B, N, H, D), dtype, 1)
    M = N // unit
    rng = np.random.default_rng(5)
    delta = rng.integers(-70000, 70000, size=(B, M) if per_inst else (M,))
    out = K.reposition(k.to(dev), torch.from_numpy(delta).to(dev), unit, style=style)
    torch.cuda.synchronize()
    p_old = np.tile(np.arange(unit), M)
    dl = delta if per_inst else np.broadcast_to(delta, (B, M))
    p_new = p_old[None] + np.repeat(dl, unit, axis=1)
    want = O.reposition(to64(k), np.broadcast_to(p_old, (B, N)), p_new, 10000.0, style, dtype)
    assert_cache_close(out, want, dtype)


def test_reposition_in_place_and_strided():
    announce("reposition_inplace_strided")
    dev = device()
    B, N, H, D = 2, 256, 8, 128
    big = rnd((B, N, H + 2, D), "bf16", 2).to(dev)        # rows padded to 10 heads
    k = big[:, :, :H, :]
    before = to64(k)
    delta = torch.arange(N // 32, dtype=torch.int64, device=dev) * 1000
    K.reposition(k, delta, 32, out=k)
    torch.cuda.synchronize()
    p_old = np.tile(np.arange(32), N // 32)
    p_new = p_old + np.repeat(np.arange(N // 32) * 1000, 32)
    want = O.reposition(before, np.broadcast_to(p_old, (B, N)), np.broadcast_to(p_new, (B, N)))
    assert_cache_close(k, want, "bf16")
    assert torch.equal(big[:, :, H:], rnd((B, N, H + 2, D), "bf16", 2)[:, :, H:].to(dev))


# --------------------------------------------------------------------------
# kvsel_score
# --------------------------------------------------------------------------
SCORE_CASES = [
    # name, dtype, B, N, H, Hq, T, D, unit
    ("stream_R4_chunks", "bf16", 3, 4096, 8, 32, 1, 128, 256),
    ("stream_R4_tokens_ragged", "bf16", 2, 3000, 4, 8, 2, 128, 1),
    ("stream_R8_ragged", "bf16", 2, 5000, 2, 16, 1, 128, 1),
    ("stream_R1", "bf16", 2, 2048, 8, 8, 1, 128, 512),
    ("tile_R16_fp32", "fp32", 1, 1024, 4, 4, 16, 64, 128),
    ("tile_R32_bf16", "bf16", 2, 2048, 4, 4, 32, 128, 512),
    ("tile_R448_ragged", "bf16", 1, 1000, 2, 14, 64, 128, 1),
    ("tile_R3_d64", "bf16", 2, 700, 2, 2, 3, 64, 1),
    ("tile_R64_fp32_d128", "fp32", 1, 1536, 2, 8, 16, 128, 96),
    # matrix-core path: bf16, >= 16 rows per kv head, segments of 64k rows
    ("mfma_R16_d64_chunks", "bf16", 1, 640, 2, 4, 8, 64, 64),
    ("mfma_R24_d64_chunks", "bf16", 2, 1536, 2, 6, 8, 64, 128),
    ("mfma_R64_chunks", "bf16", 2, 4096, 8, 16, 32, 128, 256),
    ("mfma_R128_tokens_ragged", "bf16", 2, 2000, 4, 16, 32, 128, 1),
    ("mfma_R300_two_passes_ragged", "bf16", 1, 700, 1, 10, 30, 128, 1),
    # a pass fills every wave row's first row block, then the next: 12 blocks
    # leave four single-block waves; 17 leave a second pass of one block;
    # head dim 64 with 14 blocks in four slots leaves waves of three
    ("mfma_R192_single_block_waves", "bf16", 2, 1088, 2, 24, 16, 128, 64),
    ("mfma_R272_one_block_last_pass", "bf16", 1, 900, 2, 34, 8, 128, 1),
    ("mfma_R224_d64_three_of_four", "bf16", 2, 1024, 2, 16, 14, 64, 128),
]


@pytest.mark.parametrize("case", SCORE_CASES, ids=[c[0] for c in SCORE_CASES])
def test_score(case):
    name, dtype, B, N, H, Hq, T, D, unit = case
    announce("score", case=name)
    dev = device()
    q = rnd((B, T, Hq, D), dtype, 3)
    k = rnd((B, N, H, D), dtype, 4, scale=1.5)
    scale = 1.0 / np.sqrt(D)
    rm, rs, part = K.score(q.to(dev), k.to(dev), unit, scale, row_stats=True, partials=unit > 1)
    torch.cuda.synchronize()
    m, Z, p = O.score(to64(q), to64(k), scale, unit)
    assert_rel(rm, m, 2e-3, 2e-3, "row_max")
    assert_rel(rs, Z, 2e-3, 0.0, "row_sum")
    if unit > 1:
        assert_rel(part[..., 0], p[..., 0], 2e-3, 2e-3, "m_u")
        assert_rel(part[..., 1], p[..., 1], 2e-3, 0.0, "S_u")
        # partials alone (one kernel) give the same partials
        _, _, part2 = K.score(q.to(dev), k.to(dev), unit, scale, row_stats=False, partials=True)
        assert torch.equal(part2, part)


# --------------------------------------------------------------------------
# kvsel_aggregate
# --------------------------------------------------------------------------
AGG_CASES = [
    # name, dtype, B, N, H, Hq, T, D, unit, group, signal, path
    ("chunk_mass_stats", "bf16", 4, 2048, 8, 32, 1, 128, 256, 1, "mass", "chunk"),
    ("chunk_mass_derived_group2", "bf16", 4, 2048, 4, 8, 4, 128, 128, 2, "mass", "chunk_nostats"),
    ("chunk_mass_many_rows_units", "bf16", 2, 8192, 4, 16, 16, 128, 64, 2, "mass", "chunk"),
    ("token_mass_l1", "bf16", 1, 1500, 4, 28, 4, 128, 1, 1, "mass", "token"),
    ("token_vnorm_group", "bf16", 4, 1200, 2, 8, 8, 128, 1, 4, "vnorm", "token"),
    ("token_vnorm_units_fp32", "fp32", 2, 640, 4, 4, 16, 64, 5, 2, "vnorm", "token"),
    ("token_mass_units_d64", "bf16", 2, 768, 2, 4, 3, 64, 256, 1, "mass", "token"),
    # matrix-core token path: bf16, >= 16 rows per kv head
    ("mfma_vnorm_R128_ragged_group", "bf16", 2, 1100, 4, 16, 32, 128, 1, 2, "vnorm", "token"),
    ("mfma_mass_R300_two_passes", "bf16", 1, 700, 1, 10, 30, 128, 1, 1, "mass", "token"),
    ("mfma_vnorm_R16_d64_units", "bf16", 2, 640, 2, 4, 8, 64, 5, 2, "vnorm", "token"),
    ("mfma_mass_R64", "bf16", 3, 512, 2, 16, 8, 128, 1, 1, "mass", "token"),
]


@pytest.mark.parametrize("case", AGG_CASES, ids=[c[0] for c in AGG_CASES])
def test_aggregate(case):
    name, dtype, B, N, H, Hq, T, D, unit, group, signal, path = case
    announce("aggregate", case=name)
    dev = device()
    q = rnd((B, T, Hq, D), dtype, 6).to(dev)
    k = rnd((B, N, H, D), dtype, 7, scale=1.5).to(dev)
    v = rnd((B, N, H, D), dtype, 8).to(dev)
    scale = 1.0 / np.sqrt(D)
    if path.startswith("chunk"):
        rm, rs, part = K.score(q, k, unit, scale, row_stats=True, partials=True)
        if path == "chunk":
            got = K.aggregate(unit, group, "mass", part=part, row_max=rm, row_sum=rs, k=k)
        else:
            got = K.aggregate(unit, group, "mass", part=part, cache_shape=tuple(k.shape), q=q)
    else:
        rm, rs, _ = K.score(q, k, unit, scale, row_stats=True, partials=False)
        got = K.aggregate(unit, group, signal, q=q, k=k, v=v, row_max=rm, row_sum=rs)
    torch.cuda.synchronize()
    want = O.aggregate(to64(q), to64(k), to64(v), scale, signal, unit, group)
    assert_rel(got, want, 2e-3, 0.0, "unit_score")


# --------------------------------------------------------------------------
# kvsel_topk
# --------------------------------------------------------------------------
TOPK_CASES = [
    # G, M, k, kind
    (3, 512, 64, "float"), (2, 1, 1, "float"), (4, 7, 3, "ties"), (2, 1000, 999, "ties"),
    (1, 65536, 9830, "float"), (1, 65539, 2048, "ties"), (5, 4096, 4096, "float"),
    (2, 16384, 2048, "ties_few"), (3, 2500, 1, "zeros"),
    # ~200 copies of each value: the last histogram bin holds one value, ranked
    # against itself; scores packed into a 1e-4 band; both signs
    (2, 20000, 300, "ties100"), (1, 16384, 2048, "cluster"), (3, 4096, 1000, "signed"),
    # rows re-read per pass: 19 compaction tiles with a ragged tail; several rows
    (1, 300007, 12345, "cluster"), (2, 40000, 5000, "signed"), (1, 100000, 99999, "ties100"),
    # the largest rows held in registers (32 and 64 keys per thread) and one
    # past each; ragged slices, unaligned rows when G > 1
    (1, 32768, 4000, "signed"), (2, 32769, 100, "ties"), (1, 65535, 65535, "float"),
    (3, 50001, 7, "cluster"), (1, 65536, 1, "ties_few"), (2, 65537, 30000, "signed"),
]


@pytest.mark.parametrize("G,M,k,kind", TOPK_CASES)
def test_topk(G, M, k, kind):
    announce("topk", G=G, M=M, k=k, kind=kind)
    dev = device()
    rng = np.random.default_rng(M + k)
    if kind == "float":
        s = rng.random((G, M)).astype(np.float32)
    elif kind == "ties":
        s = rng.integers(0, 50, size=(G, M)).astype(np.float32)
    elif kind == "ties_few":
        s = rng.integers(0, 3, size=(G, M)).astype(np.float32) * 0.25
    elif kind == "ties100":
        s = rng.integers(0, 100, size=(G, M)).astype(np.float32)
    elif kind == "cluster":
        s = (1.0 + 1e-4 * rng.standard_normal((G, M))).astype(np.float32)
    elif kind == "signed":
        s = rng.standard_normal((G, M)).astype(np.float32)
    else:
        s = np.where(rng.random((G, M)) < 0.5, 0.0, -0.0).astype(np.float32)
        s[:, M // 2] = 1.0
    idx, val = K.topk(torch.from_numpy(s).to(dev), k, values=True)
    torch.cuda.synchronize()
    want = O.topk(s.astype(np.float64), k)
    assert np.array_equal(idx.cpu().numpy(), want)
    assert np.array_equal(val.cpu().numpy(), np.take_along_axis(s, want, axis=1))


def test_topk_k_zero_is_noop():
    announce("topk_k0")
    dev = device()
    idx = K.topk(torch.rand(2, 10, device=dev), 0)
    torch.cuda.synchronize()
    assert idx.shape == (2, 0)


# --------------------------------------------------------------------------
# kvsel_gather
# --------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,D,unit,group", [("bf16", 128, 256, 1), ("fp32", 64, 8, 2),
                                                ("bf16", 64, 1, 1)])
def test_gather_compact(dtype, D, unit, group):
    announce("gather_compact", dtype=dtype, D=D, unit=unit, group=group)
    dev = device()
    B, H = 4, 4
    M = 40
    N = M * unit
    k = rnd((B, N, H, D), dtype, 9)
    v = rnd((B, N, H, D), dtype, 10)
    rng = np.random.default_rng(1)
    idx = np.stack([np.sort(rng.choice(M, 9, replace=False)) for _ in range(B // group)])
    gk, gv = K.gather(k.to(dev), v.to(dev), torch.from_numpy(idx).int().to(dev), unit, group)
    torch.cuda.synchronize()
    wk, wv = O.gather(to64(k), to64(v), idx, unit, group)
    assert np.array_equal(to64(gk), wk) and np.array_equal(to64(gv), wv)


@pytest.mark.parametrize("dtype,style,with_start", [("bf16", "half", False), ("bf16", "interleaved", True),
                                                    ("fp32", "half", True)])
def test_gather_align(dtype, style, with_start):
    announce("gather_align", dtype=dtype, style=style, with_start=with_start)
    dev = device()
    B, H, D, unit, M = 2, 4, 128, 64, 12
    N = M * unit
    k = rnd((B, N, H, D), dtype, 11)
    v = rnd((B, N, H, D), dtype, 12)
    idx = np.array([[0, 3, 4, 11], [1, 2, 7, 9]])
    start = np.arange(M) * 500 + 3 if with_start else np.zeros(M, np.int64)
    st = torch.from_numpy(start).to(dev) if with_start else None
    gk, gv = K.gather(k.to(dev), v.to(dev), torch.from_numpy(idx).int().to(dev), unit,
                      src_start=st, align_base=100, style=style)
    torch.cuda.synchronize()
    p_old = np.broadcast_to(np.repeat(start, unit) + np.tile(np.arange(unit), M), (B, N))
    wk = O.gather_aligned(to64(k), idx, unit, p_old, 100, 10000.0, style, dtype)
    _, wv = O.gather(to64(k), to64(v), idx, unit)
    assert_cache_close(gk, wk, dtype)
    assert np.array_equal(to64(gv), wv)


def test_gather_nested_refill():
    announce("gather_nested")
    dev = device()
    B, H, D, l, m = 2, 4, 128, 8, 300
    l1k, l1v = rnd((B, m, H, D), "bf16", 13), rnd((B, m, H, D), "bf16", 14)
    l2k, l2v = rnd((B, m * l, H, D), "bf16", 15), rnd((B, m * l, H, D), "bf16", 16)
    rng = np.random.default_rng(3)
    idx = np.stack([np.sort(rng.choice(m, 37, replace=False)) for _ in range(B)])
    gk, gv = K.gather(l2k.to(dev), l2v.to(dev), torch.from_numpy(idx).int().to(dev), l,
                      proxy_k=l1k.to(dev), proxy_v=l1v.to(dev))
    torch.cuda.synchronize()
    for b in range(B):
        assert np.array_equal(to64(gk[b]), O.refill_nested(to64(l1k[b]), to64(l2k[b]), idx[b], l))
        assert np.array_equal(to64(gv[b]), O.refill_nested(to64(l1v[b]), to64(l2v[b]), idx[b], l))


# --------------------------------------------------------------------------
# kvsel_decode_attn
# --------------------------------------------------------------------------
DECODE_CASES = [
    # name, dtype, B, segs N, H, Hq, T, D
    ("stream_R4", "bf16", 3, (1300,), 8, 32, 1, 128),
    ("stream_R4_two_segs", "bf16", 2, (1024, 77), 8, 32, 1, 128),
    ("stream_R2_T2", "bf16", 2, (600,), 4, 4, 2, 128),
    # rows per kv head padded to the next of 1, 2, 4
    ("stream_R3_padded_two_segs", "bf16", 2, (700, 33), 8, 24, 1, 128),
    # 5 to 15 rows: the matrix cores, one 16-row block
    ("mfma_R7_one_block", "bf16", 3, (2560,), 4, 28, 1, 128),
    ("mfma_R6_T3_one_block", "bf16", 2, (900,), 2, 4, 3, 128),
    ("mfma_R5_d64_two_segs", "bf16", 2, (300, 70), 2, 10, 1, 64),
    ("tile_R16_fp32", "fp32", 1, (256,), 4, 4, 16, 64),
    ("tile_R448_two_segs", "bf16", 1, (700, 600), 4, 28, 64, 128),
    ("tile_R32_bf16", "bf16", 1, (1100,), 4, 4, 32, 128),
    ("tile_R3_d64", "bf16", 2, (513, 5), 2, 2, 3, 64),
    # matrix-core path: bf16, >= 16 rows per kv head
    ("mfma_R16_d64_two_segs", "bf16", 2, (700, 77), 2, 4, 8, 64),
    ("mfma_R128_ragged", "bf16", 1, (1300,), 4, 16, 32, 128),
    ("mfma_R300_d64_three_passes", "bf16", 1, (530, 40), 1, 10, 30, 64),
    # two row blocks per wave: one pass with idle waves, a segment shorter than a tile
    ("mfma_R224_one_pass_short_seg", "bf16", 2, (1030, 5), 4, 28, 32, 128),
    ("mfma_R200_d64_one_pass", "bf16", 1, (2100,), 2, 10, 40, 64),
    # a pass fills every wave's first row block, then the second: 12 blocks
    # leave four waves one block; 17 leave a second pass of one block (seven
    # waves without query rows); 32 fill two passes
    ("mfma_R192_one_pass_four_single", "bf16", 2, (900,), 2, 24, 16, 128),
    ("mfma_R272_one_block_last_pass", "bf16", 1, (1500, 40), 4, 68, 16, 128),
    ("mfma_R512_two_full_passes", "bf16", 1, (800,), 2, 32, 32, 128),
]


def strided(t, pad_heads, pad_rows):
    """t ([B][N][H][D]) as a view with padded rows (stride_n = (H + pad_heads) * D)
    and padded instances (pad_rows extra rows each): the layout of a cache
    slice inside a larger store."""
    B, N, H, D = t.shape
    big = torch.zeros((B, N + pad_rows, H + pad_heads, D), dtype=t.dtype, device=t.device)
    big[:, :N, :H] = t
    return big[:, :N, :H]


# the same calls on strided caches: the tall matrix-core plan (buffer-resource
# loads at byte offsets of the row stride), the streaming and four-wave plans
STRIDED_DECODE_CASES = [
    # name, B, segs N, H, Hq, T, pad_heads, pad_rows
    ("mfma_R448_strided", 2, (700, 130), 4, 28, 64, 3, 5),
    ("mfma_R64_strided", 2, (900,), 2, 8, 16, 1, 64),
    ("stream_R4_strided", 3, (1030,), 8, 32, 1, 2, 9),
]


@pytest.mark.parametrize("case", STRIDED_DECODE_CASES, ids=[c[0] for c in STRIDED_DECODE_CASES])
def test_decode_strided(case):
    name, B, Ns, H, Hq, T, ph, pr = case
    announce("decode_strided", case=name)
    dev = device()
    D = 128
    q = rnd((B, T, Hq, D), "bf16", 27)
    segs = [(rnd((B, n, H, D), "bf16", 28 + i, 1.5), rnd((B, n, H, D), "bf16", 50 + i))
            for i, n in enumerate(Ns)]
    views = [(strided(a.to(dev), ph, pr), strided(b.to(dev), ph, pr)) for a, b in segs]
    assert views[0][0].stride(1) == (H + ph) * D and not views[0][0].is_contiguous()
    o, lse = K.decode_attn(q.to(dev), views)
    torch.cuda.synchronize()
    wo, wl = O.decode_attention(to64(q), [(to64(a), to64(b)) for a, b in segs], 1.0 / np.sqrt(D))
    assert_rel(o, wo, 0.0, 5e-3, "o")
    assert_rel(lse, wl, 0.0, 2e-3, "lse")


@pytest.mark.parametrize("case", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_decode(case):
    name, dtype, B, Ns, H, Hq, T, D = case
    announce("decode", case=name)
    dev = device()
    q = rnd((B, T, Hq, D), dtype, 17)
    segs = [(rnd((B, n, H, D), dtype, 18 + i, 1.5), rnd((B, n, H, D), dtype, 40 + i))
            for i, n in enumerate(Ns)]
    o, lse = K.decode_attn(q.to(dev), [(a.to(dev), b.to(dev)) for a, b in segs])
    torch.cuda.synchronize()
    wo, wl = O.decode_attention(to64(q), [(to64(a), to64(b)) for a, b in segs], 1.0 / np.sqrt(D))
    assert_rel(o, wo, 0.0, 5e-3, "o")
    assert_rel(lse, wl, 0.0, 2e-3, "lse")


# --------------------------------------------------------------------------
# kvsel_gather_decode (refill + final attention pass in one call)
# --------------------------------------------------------------------------
GD_CASES = [
    # name, dtype, B, H, Hq, T, D, unit, M, kept, idx_group, extra N list
    ("fused_R4_chunks", "bf16", 3, 8, 32, 1, 128, 256, 12, 5, 1, ()),
    ("fused_R2_tokens_group_extra", "bf16", 4, 4, 8, 1, 128, 1, 1000, 300, 2, (77,)),
    ("fused_R8_ragged_two_extra", "bf16", 2, 2, 16, 1, 128, 3, 400, 171, 1, (513, 40)),
    ("fused_R7_padded", "bf16", 2, 4, 28, 1, 128, 512, 8, 5, 1, ()),
    ("fused_R5_padded_extra", "bf16", 3, 1, 5, 1, 128, 64, 20, 7, 1, (130,)),
    ("tile_R448_refill_extra", "bf16", 1, 4, 28, 16, 128, 8, 300, 37, 1, (300,)),
    ("tile_fp32_d64", "fp32", 2, 4, 4, 16, 64, 64, 10, 3, 1, ()),
    ("fused_k0_extra_only", "bf16", 2, 8, 32, 1, 128, 256, 4, 0, 1, (600,)),
]


@pytest.mark.parametrize("case", GD_CASES, ids=[c[0] for c in GD_CASES])
def test_gather_decode(case):
    name, dtype, B, H, Hq, T, D, unit, M, kept, group, extra_n = case
    announce("gather_decode", case=name)
    dev = device()
    N = M * unit
    q = rnd((B, T, Hq, D), dtype, 50)
    k = rnd((B, N, H, D), dtype, 51, 1.5)
    v = rnd((B, N, H, D), dtype, 52)
    extra = [(rnd((B, n, H, D), dtype, 60 + i, 1.5), rnd((B, n, H, D), dtype, 70 + i))
             for i, n in enumerate(extra_n)]
    rng = np.random.default_rng(kept + M)
    idx = np.stack([np.sort(rng.choice(M, kept, replace=False)) for _ in range(B // group)])
    idx_t = torch.from_numpy(idx).int().to(dev).reshape(B // group, kept)
    kd, vd, o, lse = K.gather_decode(q.to(dev), k.to(dev), v.to(dev), idx_t, unit, group,
                                     extra=[(a.to(dev), b.to(dev)) for a, b in extra])
    torch.cuda.synchronize()
    wk, wv = O.gather(to64(k), to64(v), idx, unit, group)
    assert np.array_equal(to64(kd), wk) and np.array_equal(to64(vd), wv)
    segs = [(to64(a), to64(b)) for a, b in extra] + ([(wk, wv)] if kept else [])
    wo, wl = O.decode_attention(to64(q), segs, 1.0 / np.sqrt(D))
    assert_rel(o, wo, 0.0, 5e-3, "o")
    assert_rel(lse, wl, 0.0, 2e-3, "lse")
    # the separate calls give the same output (the same kernel where the plain
    # decode also streams; from 5 rows per kv head it runs on the matrix cores
    # with bf16 weights, so the two agree to the parity tolerance)
    segs_d = [(a.to(dev), b.to(dev)) for a, b in extra] + ([(kd, vd)] if kept else [])
    o2, lse2 = K.decode_attn(q.to(dev), segs_d)
    torch.cuda.synchronize()
    same_kernel = not (dtype == "bf16" and (Hq // H) * T >= 5)
    assert_rel(o2, to64(o), 0.0, 1e-5 if same_kernel else 5e-3, "o vs separate calls")


# --------------------------------------------------------------------------
# kvsel_score_reposition (re-position + score, fused where the shape allows)
# --------------------------------------------------------------------------
SR_CASES = [
    # name, dtype, B, N, H, Hq, T, D, unit (score), rot_unit, style, per_inst, keep
    ("fused_chunks_half_nokeep", "bf16", 1, 4096, 4, 8, 8, 128, 512, 512, "half", False, False),
    ("fused_tokens_half_keep_ragged", "bf16", 2, 2112, 2, 8, 16, 128, 1, 64, "half", True, True),
    ("fused_tokens_interleaved_d64", "bf16", 2, 1024, 2, 4, 8, 64, 1, 256, "interleaved", False, True),
    ("fused_R300_passes_keep", "bf16", 1, 1280, 1, 10, 30, 128, 1, 128, "half", False, True),
    ("stream_R4_nokeep_uses_ws", "bf16", 2, 2048, 8, 32, 1, 128, 256, 256, "half", False, False),
    ("fp32_two_pass_keep", "fp32", 1, 1024, 4, 4, 16, 64, 128, 128, "half", False, True),
]


@pytest.mark.parametrize("case", SR_CASES, ids=[c[0] for c in SR_CASES])
def test_score_reposition(case):
    name, dtype, B, N, H, Hq, T, D, unit, rot, style, per_inst, keep = case
    announce("score_reposition", case=name)
    dev = device()
    q = rnd((B, T, Hq, D), dtype, 80).to(dev)
    k = rnd((B, N, H, D), dtype, 81, 1.5).to(dev)
    M = N // rot
    rng = np.random.default_rng(9)
    delta = torch.from_numpy(rng.integers(0, 66000, size=(B, M) if per_inst else (M,))).to(dev)
    chunk = unit > 1
    k_out = torch.empty_like(k) if keep else None
    rm, rs, part = K.score_reposition(q, k, delta, rot, unit, k_out=k_out, row_stats=True,
                                      partials=chunk, style=style)
    # reference: the two separate calls
    k_ref = K.reposition(k, delta, rot, style=style)
    rm2, rs2, part2 = K.score(q, k_ref, unit, row_stats=True, partials=chunk)
    torch.cuda.synchronize()
    assert torch.equal(rm, rm2) and torch.equal(rs, rs2)
    if chunk:
        assert torch.equal(part, part2)
    if keep:
        assert torch.equal(k_out, k_ref)
    # and the oracle on the re-positioned keys
    p_old = np.tile(np.arange(rot), M)
    dl = delta.cpu().numpy() if per_inst else np.broadcast_to(delta.cpu().numpy(), (B, M))
    p_new = p_old[None] + np.repeat(dl, rot, axis=1)
    want_k = O.reposition(to64(k), np.broadcast_to(p_old, (B, N)), p_new, 10000.0, style, dtype)
    m, Z, _ = O.score(to64(q), want_k, 1.0 / np.sqrt(D), 1)
    assert_rel(rm, m, 2e-3, 2e-3, "row_max")
    assert_rel(rs, Z, 2e-3, 0.0, "row_sum")
