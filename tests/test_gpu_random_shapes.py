"""Seeded random shapes for the scorer (plain, with re-positioning fused, and
over listed units), the aggregate, the top-k, the gather, the decode attention (plain and with the
refill fused) and the index-based causal attention, against the oracle: rows per kv head drawn across
every plan boundary (the streaming kernels up to 8 rows, one 16-row block,
four-wave plans up to 128 rows, eight-wave plans of two row blocks, several
row passes), head dim 64 and 128, bf16 and fp32, ragged cache lengths, units
of 1 to 256 rows, instance groups, one or two decode segments, top-k rows of
1 to 120,000 scores with heavy ties.  Each case draws its shape from its own
seed, so a failure names a shape that reproduces.  Tolerances as in the
per-call tests: scores within relative 2e-3, decode outputs within 5e-3
absolute, indices, values and copies bit-exact.
"""

import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import announce, assert_rel, device
from oracle.pipeline import to64
from query_guided_kv_amd import kvsel as K

pytestmark = pytest.mark.gpu

TD = {"bf16": torch.bfloat16, "fp32": torch.float32}
N_CASES = 64


def rnd(shape, dtype, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (scale * torch.randn(shape, generator=g)).to(TD[dtype])


def draw(seed: int) -> dict:
    """A shape: rows per kv head (query heads per kv head x tokens) spread
    over 1 .. 448, with the oracle's work kept to a few hundred MFLOP."""
    rng = np.random.default_rng(1000 + seed)
    dtype = "fp32" if rng.random() < 0.15 else "bf16"
    D = int(rng.choice([64, 128, 128]))
    H = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 4, 7, 8]))
    rows = int(rng.choice([1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 64, 100, 128, 160, 224, 300, 448]))
    T = max(1, rows // G)
    B = int(rng.choice([1, 2]))
    unit = int(rng.choice([1, 64, 128, 256]))
    budget = 4e8 / (B * H * G * T * D)          # cached rows the oracle can afford
    n_units = max(1, int(rng.integers(1, max(2, int(budget // unit) + 1))))
    n_units = min(n_units, max(1, 3000 // unit))
    N = unit * n_units if unit > 1 else int(rng.integers(33, max(34, min(3000, int(budget)))))
    split = int(rng.integers(1, N)) if N > 1 and rng.random() < 0.5 else N
    return dict(dtype=dtype, D=D, H=H, G=G, T=T, B=B, N=N, unit=unit, split=split)


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_score(seed):
    c = draw(seed)
    announce("random_score", seed=seed, **c)
    dev = device()
    B, N, H, D, T, Hq = c["B"], c["N"], c["H"], c["D"], c["T"], c["H"] * c["G"]
    q = rnd((B, T, Hq, D), c["dtype"], 2 * seed)
    k = rnd((B, N, H, D), c["dtype"], 2 * seed + 1, scale=1.5)
    scale = 1.0 / np.sqrt(D)
    unit = c["unit"]
    rm, rs, part = K.score(q.to(dev), k.to(dev), unit, scale, row_stats=True, partials=unit > 1)
    torch.cuda.synchronize()
    m, Z, p = O.score(to64(q), to64(k), scale, unit)
    assert_rel(rm, m, 2e-3, 2e-3, "row_max")
    assert_rel(rs, Z, 2e-3, 0.0, "row_sum")
    if unit > 1:
        assert_rel(part[..., 0], p[..., 0], 2e-3, 2e-3, "m_u")
        assert_rel(part[..., 1], p[..., 1], 2e-3, 0.0, "S_u")


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_decode(seed):
    c = draw(seed)
    announce("random_decode", seed=seed, **c)
    dev = device()
    B, N, H, D, T, Hq = c["B"], c["N"], c["H"], c["D"], c["T"], c["H"] * c["G"]
    q = rnd((B, T, Hq, D), c["dtype"], 3 * seed)
    k = rnd((B, N, H, D), c["dtype"], 3 * seed + 1)
    v = rnd((B, N, H, D), c["dtype"], 3 * seed + 2)
    # one segment, or the cache cut in two at a random row (the second
    # segment a separate allocation, as a refilled part would be)
    s = c["split"]
    pairs = [(k[:, :s].contiguous(), v[:, :s].contiguous())]
    if s < N:
        pairs.append((k[:, s:].contiguous(), v[:, s:].contiguous()))
    scale = 1.0 / np.sqrt(D)
    o, lse = K.decode_attn(q.to(dev), [(a.to(dev), b.to(dev)) for a, b in pairs], scale)
    torch.cuda.synchronize()
    want_o, want_lse = O.decode_attention(to64(q), [(to64(a), to64(b)) for a, b in pairs], scale)
    assert_rel(o, want_o, 0.0, 5e-3, "decode output")
    assert_rel(lse, want_lse, 0.0, 2e-3, "lse")


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_aggregate(seed):
    """Per-unit attention mass or mass x |v| (token path), or the chunk
    combine of the scorer's partials (chunk path), grouped over instances."""
    c = draw(seed)
    rng = np.random.default_rng(2000 + seed)
    signal = "vnorm" if rng.random() < 0.5 else "mass"
    unit = c["unit"] if c["unit"] > 1 or rng.random() < 0.5 else int(rng.choice([1, 5]))
    path = "chunk" if unit % 64 == 0 and signal == "mass" and rng.random() < 0.5 else "token"
    B, H, D, T, Hq = c["B"], c["H"], c["D"], c["T"], c["H"] * c["G"]
    N = c["N"] - c["N"] % unit if unit > 1 else c["N"]
    group = B if rng.random() < 0.5 else 1
    announce("random_aggregate", seed=seed, signal=signal, path=path, unit=unit, N=N, group=group,
             **{k: c[k] for k in ("dtype", "D", "H", "G", "T", "B")})
    dev = device()
    q = rnd((B, T, Hq, D), c["dtype"], 5 * seed).to(dev)
    k = rnd((B, N, H, D), c["dtype"], 5 * seed + 1, scale=1.5).to(dev)
    v = rnd((B, N, H, D), c["dtype"], 5 * seed + 2).to(dev)
    scale = 1.0 / np.sqrt(D)
    if path == "chunk":
        rm, rs, part = K.score(q, k, unit, scale, row_stats=True, partials=True)
        got = K.aggregate(unit, group, "mass", part=part, row_max=rm, row_sum=rs, k=k)
    else:
        rm, rs, _ = K.score(q, k, unit, scale, row_stats=True, partials=False)
        got = K.aggregate(unit, group, signal, q=q, k=k, v=v, row_max=rm, row_sum=rs)
    torch.cuda.synchronize()
    want = O.aggregate(to64(q), to64(k), to64(v), scale, signal, unit, group)
    assert_rel(got, want, 2e-3, 0.0, "unit_score")


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_topk(seed):
    """Rows of random length and k, with continuous scores, heavy ties or
    values packed into a narrow band: indices and values bit-exact."""
    rng = np.random.default_rng(3000 + seed)
    G = int(rng.integers(1, 5))
    M = int(rng.choice([int(rng.integers(1, 300)), int(rng.integers(300, 20000)),
                        int(rng.integers(20000, 120000))]))
    k = int(rng.integers(0, M + 1))
    kind = str(rng.choice(["float", "ties", "band"]))
    announce("random_topk", seed=seed, G=G, M=M, k=k, kind=kind)
    if kind == "float":
        s = rng.standard_normal((G, M)).astype(np.float32)
    elif kind == "ties":
        s = rng.integers(0, int(rng.integers(2, 200)), size=(G, M)).astype(np.float32)
    else:
        s = (3.0 + 1e-5 * rng.standard_normal((G, M))).astype(np.float32)
    dev = device()
    idx, val = K.topk(torch.from_numpy(s).to(dev), k, values=True)
    torch.cuda.synchronize()
    want = O.topk(s.astype(np.float64), k)
    assert np.array_equal(idx.cpu().numpy(), want)
    assert np.array_equal(val.cpu().numpy(), np.take_along_axis(s, want, axis=1))


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_gather(seed):
    """Kept units of random length gathered into the compact layout: bit-exact."""
    c = draw(seed)
    rng = np.random.default_rng(4000 + seed)
    unit = int(rng.choice([1, 3, 64, 256]))
    M = int(rng.integers(1, max(2, 3000 // unit)))
    group = c["B"] if rng.random() < 0.5 else 1
    kept = int(rng.integers(1, M + 1))
    B, H, D = c["B"], c["H"], c["D"]
    N = M * unit
    announce("random_gather", seed=seed, unit=unit, M=M, kept=kept, group=group,
             **{k: c[k] for k in ("dtype", "D", "H", "B")})
    k = rnd((B, N, H, D), c["dtype"], 7 * seed)
    v = rnd((B, N, H, D), c["dtype"], 7 * seed + 1)
    idx = np.stack([np.sort(rng.choice(M, kept, replace=False)) for _ in range(B // group)])
    dev = device()
    gk, gv = K.gather(k.to(dev), v.to(dev), torch.from_numpy(idx).int().to(dev), unit, group)
    torch.cuda.synchronize()
    wk, wv = O.gather(to64(k), to64(v), idx, unit, group)
    assert np.array_equal(to64(gk), wk) and np.array_equal(to64(gv), wv)


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_score_reposition(seed):
    """Re-positioning fused into the scorer: the same row statistics, bit for
    bit, as re-positioning then scoring (and the same K' where it is kept),
    and the oracle on the re-positioned keys."""
    c = draw(seed)
    rng = np.random.default_rng(5000 + seed)
    rot = int(rng.choice([1, 8, 64, 128, 256, 512]))
    M = int(rng.integers(1, max(2, 3000 // rot)))
    N = M * rot
    style = str(rng.choice(["half", "interleaved"]))
    per_inst = bool(rng.random() < 0.5)
    keep = bool(rng.random() < 0.5)
    B, H, D, T, Hq = c["B"], c["H"], c["D"], c["T"], c["H"] * c["G"]
    announce("random_score_reposition", seed=seed, rot=rot, N=N, style=style, per_inst=per_inst,
             keep=keep, **{k: c[k] for k in ("dtype", "D", "H", "G", "T", "B")})
    dev = device()
    q = rnd((B, T, Hq, D), c["dtype"], 11 * seed).to(dev)
    k = rnd((B, N, H, D), c["dtype"], 11 * seed + 1, 1.5).to(dev)
    delta = torch.from_numpy(rng.integers(0, 66000, size=(B, M) if per_inst else (M,))).to(dev)
    k_out = torch.empty_like(k) if keep else None
    rm, rs, _ = K.score_reposition(q, k, delta, rot, 1, k_out=k_out, row_stats=True,
                                   partials=False, style=style)
    k_ref = K.reposition(k, delta, rot, style=style)
    rm2, rs2, _ = K.score(q, k_ref, 1, row_stats=True, partials=False)
    torch.cuda.synchronize()
    assert torch.equal(rm, rm2) and torch.equal(rs, rs2)
    if keep:
        assert torch.equal(k_out, k_ref)
    p_old = np.tile(np.arange(rot), M)
    dl = delta.cpu().numpy() if per_inst else np.broadcast_to(delta.cpu().numpy(), (B, M))
    p_new = p_old[None] + np.repeat(dl, rot, axis=1)
    want_k = O.reposition(to64(k), np.broadcast_to(p_old, (B, N)), p_new, 10000.0, style,
                          c["dtype"])
    m, Z, _ = O.score(to64(q), want_k, 1.0 / np.sqrt(D), 1)
    assert_rel(rm, m, 2e-3, 2e-3, "row_max")
    assert_rel(rs, Z, 2e-3, 0.0, "row_sum")


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_gather_decode(seed):
    """Refill and decode in one call: the compact cache bit-exact, the
    attention over it (after any extra segments) within tolerance."""
    c = draw(seed)
    rng = np.random.default_rng(6000 + seed)
    unit = int(rng.choice([1, 3, 64, 256]))
    M = int(rng.integers(1, max(2, 2500 // unit)))
    kept = int(rng.integers(0, M + 1))
    group = c["B"] if rng.random() < 0.5 else 1
    n_extra = int(rng.integers(0 if kept else 1, 3))
    extra_n = [int(rng.integers(1, 600)) for _ in range(n_extra)]
    B, H, D, T, Hq = c["B"], c["H"], c["D"], c["T"], c["H"] * c["G"]
    N = M * unit
    announce("random_gather_decode", seed=seed, unit=unit, M=M, kept=kept, group=group,
             extra=extra_n, **{k: c[k] for k in ("dtype", "D", "H", "G", "T", "B")})
    dev = device()
    q = rnd((B, T, Hq, D), c["dtype"], 13 * seed)
    k = rnd((B, N, H, D), c["dtype"], 13 * seed + 1, 1.5)
    v = rnd((B, N, H, D), c["dtype"], 13 * seed + 2)
    extra = [(rnd((B, n, H, D), c["dtype"], 13 * seed + 3 + 2 * i, 1.5),
              rnd((B, n, H, D), c["dtype"], 13 * seed + 4 + 2 * i)) for i, n in enumerate(extra_n)]
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


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_index_attn(seed):
    """Selected tokens attending causally to the context, positions anywhere
    (some before the first row, some past the last)."""
    rng = np.random.default_rng(7000 + seed)
    B = int(rng.integers(1, 3))
    H = int(rng.choice([1, 2, 4]))
    Hq = H * int(rng.choice([1, 4, 7]))
    D = int(rng.choice([64, 128, 128]))
    N = int(rng.integers(1, 2500))
    S = int(rng.integers(1, 300))
    announce("random_index_attn", seed=seed, B=B, H=H, Hq=Hq, D=D, N=N, S=S)
    dev = device()
    g = torch.Generator().manual_seed(8000 + seed)
    q = torch.randn((B, S, Hq, D), generator=g).to(torch.bfloat16)
    k = (1.5 * torch.randn((B, N, H, D), generator=g)).to(torch.bfloat16)
    v = torch.randn((B, N, H, D), generator=g).to(torch.bfloat16)
    pos = rng.integers(-3, N + 3, size=(B, S))
    if rng.random() < 0.5:
        pos = np.sort(pos, axis=1)
    pos = pos.astype(np.int32)
    o, lse = K.index_attn(q.to(dev), k.to(dev), v.to(dev), torch.from_numpy(pos).to(dev))
    torch.cuda.synchronize()
    wo, wl = O.index_causal_attention(to64(q), to64(k), to64(v), pos, 1 / np.sqrt(D))
    assert_rel(o, wo, 0.0, 5e-3, "output")
    fin = np.isfinite(wl)
    got_l = lse.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isfinite(got_l), fin)
    assert_rel(got_l[fin], wl[fin], 0.0, 5e-3, "lse")


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_score_units(seed):
    """Listed units of a cache (repeats allowed), re-positioned to random
    positions or not, scored in place: row statistics and per-unit partials
    against the oracle on the concatenated, re-positioned copy."""
    c = draw(seed)
    rng = np.random.default_rng(9000 + seed)
    U = int(rng.choice([64, 96, 128, 256, 512]))
    n_src = int(rng.integers(1, max(2, 2500 // U)))
    n = int(rng.integers(1, 2 * n_src + 1))
    dmode = str(rng.choice(["none", "shared", "inst"]))
    style = str(rng.choice(["half", "interleaved"]))
    B, H, D, T, Hq = c["B"], c["H"], c["D"], c["T"], c["H"] * c["G"]
    announce("random_score_units", seed=seed, U=U, n_src=n_src, n=n, dmode=dmode, style=style,
             **{k: c[k] for k in ("dtype", "D", "H", "G", "T", "B")})
    dev = device()
    k = rnd((B, n_src * U, H, D), c["dtype"], 17 * seed, 1.5)
    q = rnd((B, T, Hq, D), c["dtype"], 17 * seed + 1)
    units = rng.integers(0, n_src, size=(B, n))
    if dmode == "shared":
        delta = rng.integers(0, 60000, size=(n,))
    elif dmode == "inst":
        delta = rng.integers(-40000, 40000, size=(B, n))
    else:
        delta = None
    scale = 1.0 / np.sqrt(D)
    rm, rs, part = K.score_units(q.to(dev), k.to(dev), torch.from_numpy(units.astype(np.int32)).to(dev),
                                 U, delta=None if delta is None else torch.from_numpy(delta).to(dev),
                                 scale=scale, style=style)
    torch.cuda.synchronize()
    k64 = to64(k)
    rows = (units[:, :, None] * U + np.arange(U)[None, None, :]).reshape(B, n * U)
    concat = np.stack([k64[b, rows[b]] for b in range(B)])
    if delta is not None:
        p_old = np.tile(np.arange(U), n)
        p_new = p_old[None] + np.repeat(np.broadcast_to(delta, (B, n)), U, axis=1)
        concat = O.reposition(concat, np.broadcast_to(p_old, (B, n * U)), p_new, 10000.0, style,
                              c["dtype"])
    m, Z, p = O.score(to64(q), concat, scale, U)
    assert_rel(rm, m, 2e-3, 2e-3, "row_max")
    assert_rel(rs, Z, 2e-3, 0.0, "row_sum")
    assert_rel(part[..., 0], p[..., 0], 2e-3, 2e-3, "m_u")
    assert_rel(part[..., 1], p[..., 1], 2e-3, 0.0, "S_u")
