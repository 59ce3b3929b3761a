"""The C ABI: library loads, exports every declared symbol, validates arguments.

CPU only: every call here fails validation before anything would be enqueued,
so no GPU is touched.  Device pointers are fake (aligned) integers.
"""

import ctypes
import os
import re

import pytest

from query_guided_kv_amd import kvsel as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvsel.h")

OK, NULL, SHAPE, DTYPE, UNSUP, WS = 0, -1, -2, -3, -4, -5
FAKE = 0x10000            # aligned, never dereferenced
MISALIGNED = 0x10008


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(K.LIB_PATH):
        from query_guided_kv_amd import build
        build.build()
    return K.load()


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvsel_[a-z_]+)\s*\(", text)))


def test_header_declares_the_six_calls():
    syms = declared_symbols()
    for name in ["kvsel_reposition", "kvsel_score", "kvsel_aggregate", "kvsel_topk",
                 "kvsel_gather", "kvsel_decode_attn"]:
        assert name in syms


def test_every_declared_symbol_is_exported(lib):
    for name in declared_symbols():
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.kvsel_version() == 100
    assert lib.kvsel_status_str(0) == b"ok"
    for code in (NULL, SHAPE, DTYPE, UNSUP, WS, -6):
        assert lib.kvsel_status_str(code) not in (b"ok", b"unknown status")
    assert lib.kvsel_status_str(-99) == b"unknown status"


def cache(B=2, N=1024, H=8, D=128, dtype=K.BF16, stride_n=None, stride_b=None):
    sn = H * D if stride_n is None else stride_n
    sb = N * sn if stride_b is None else stride_b
    return K.Cache(B, N, H, D, sb, sn, dtype)


def test_reposition_validation(lib):
    d = ctypes.c_void_p(FAKE)
    f = lambda kc, unit=64, style=0, base=10000.0, kin=FAKE, delta=FAKE: lib.kvsel_reposition(
        kin and ctypes.c_void_p(kin), d, kc, unit, delta and ctypes.c_void_p(delta), 0, base, style, None)
    assert f(cache(), kin=0) == NULL
    assert f(cache(), delta=0) == NULL
    assert f(cache(), kin=MISALIGNED) == UNSUP
    assert f(cache(dtype=7)) == DTYPE
    assert f(cache(D=96)) == UNSUP
    assert f(cache(), unit=100) == SHAPE          # 1024 % 100 != 0
    assert f(cache(), unit=0) == SHAPE
    assert f(cache(), style=5) == SHAPE
    assert f(cache(), base=0.5) == SHAPE
    assert f(cache(stride_n=1000)) == SHAPE       # < H*D
    assert f(cache(stride_n=1028)) == UNSUP       # not a multiple of 8
    assert f(cache(B=0)) == SHAPE
    assert b"unit_len" in lib.kvsel_last_error() or True


def test_score_validation(lib):
    p = ctypes.c_void_p(FAKE)
    kc = cache()
    call = lambda T=1, Hq=32, unit=256, rm=FAKE, rs=FAKE, part=FAKE, ws=None, wsb=0, kc=kc: lib.kvsel_score(
        p, T, Hq, p, kc, 0.088, unit, rm and ctypes.c_void_p(rm), rs and ctypes.c_void_p(rs),
        part and ctypes.c_void_p(part), ws, wsb, None)
    assert call(Hq=30) == SHAPE                   # not a multiple of H
    assert call(T=0) == SHAPE
    assert call(unit=300) == SHAPE
    assert call(rm=0) == NULL                      # row_max without row_sum
    assert call(rm=0, rs=0, part=0) == NULL        # nothing requested
    assert call(unit=1) == SHAPE                   # partials need units
    # row statistics without partials need a workspace
    need = lib.kvsel_score_workspace(2, 1024, 32, 1, 1, 1, 0)
    assert need == 2 * 32 * 1 * (1024 // 256) * 2 * 4
    assert call(unit=1, part=0) == WS
    assert call(unit=1, part=0, ws=ctypes.c_void_p(FAKE), wsb=need - 1) == WS
    assert lib.kvsel_score_workspace(2, 1024, 32, 1, 256, 1, 1) == 0


def test_aggregate_validation(lib):
    p = ctypes.c_void_p(FAKE)
    kc = cache()
    call = lambda sig=0, unit=256, group=1, part=FAKE, rm=FAKE, rs=FAKE, out=FAKE, q=FAKE, ws=None, wsb=0: lib.kvsel_aggregate(
        q and ctypes.c_void_p(q), 1, 32, p, p, kc, 0.088, rm and ctypes.c_void_p(rm),
        rs and ctypes.c_void_p(rs), part and ctypes.c_void_p(part), sig, unit, group,
        out and ctypes.c_void_p(out), ws, wsb, None)
    assert call(sig=3) == SHAPE
    assert call(group=3) == SHAPE                  # 2 % 3 != 0
    assert call(out=0) == NULL
    assert call(rm=0) == NULL
    assert call(rm=0, rs=0) == WS                  # derives row stats: needs workspace
    assert call(part=0, rm=0, rs=0, ws=ctypes.c_void_p(FAKE), wsb=1 << 30) == NULL  # token path needs stats
    assert call(part=0, q=0, ws=ctypes.c_void_p(FAKE), wsb=1 << 30) == NULL
    assert lib.kvsel_aggregate_workspace(2, 1024, 32, 1, 1, 0, 1) == 2 * 1024 * 4
    # chunk path: derived row stats (2 x B*Hq*T) + row-chunk sums ((ceil(B*Hq*T/64) + B) x M)
    assert lib.kvsel_aggregate_workspace(2, 1024, 32, 1, 256, 1, 0) == (2 * 2 * 32 + (1 + 2) * 4) * 4
    assert lib.kvsel_aggregate_workspace(2, 1024, 32, 1, 256, 1, 1) == (1 + 2) * 4 * 4


def test_topk_validation(lib):
    p = ctypes.c_void_p(FAKE)
    assert lib.kvsel_topk(None, 1, 10, 2, p, None, None) == NULL
    assert lib.kvsel_topk(p, 1, 10, 11, p, None, None) == SHAPE
    assert lib.kvsel_topk(p, 1, 10, -1, p, None, None) == SHAPE
    assert lib.kvsel_topk(p, 0, 10, 1, p, None, None) == SHAPE
    assert lib.kvsel_topk(p, 1, 1 << 31, 1, p, None, None) == SHAPE
    assert lib.kvsel_topk(p, 1, 10, 0, None, None, None) == OK      # k == 0: no-op
    assert lib.kvsel_topk(p, 1, 10, 3, None, None, None) == NULL


def test_gather_validation(lib):
    p = ctypes.c_void_p(FAKE)
    kc = cache()
    call = lambda k=4, unit=256, group=1, v_src=FAKE, v_dst=FAKE, align=-1, style=0, proxy=None, kp=None, vp=None: lib.kvsel_gather(
        p, v_src and ctypes.c_void_p(v_src), kc, unit, p, k, group, None, align, 10000.0, style,
        kp, vp, proxy, p, v_dst and ctypes.c_void_p(v_dst), None)
    assert call(k=5) == SHAPE                      # M = 4
    assert call(v_dst=0) == NULL
    assert call(group=3) == SHAPE
    assert call(unit=3) == SHAPE
    assert call(align=0, style=9) == SHAPE
    bad = cache(N=5)
    assert call(proxy=ctypes.pointer(bad), kp=p, vp=p) == SHAPE          # proxy N != M
    good = cache(N=4)
    assert call(proxy=ctypes.pointer(good), kp=p, vp=None) == NULL       # v_proxy missing
    assert call(proxy=ctypes.pointer(good), kp=p, vp=p, align=0) == UNSUP
    assert call(k=0, v_src=0, v_dst=0) == OK       # nothing to copy


def test_decode_validation(lib):
    p = ctypes.c_void_p(FAKE)
    seg = (K.Segment * 2)(K.Segment(FAKE, FAKE, cache()), K.Segment(FAKE, FAKE, cache(H=4)))
    out = ctypes.c_void_p(FAKE)
    assert lib.kvsel_decode_attn(p, 1, 32, 0.1, seg, 2, out, None, p, 1 << 40, None) == SHAPE
    assert lib.kvsel_decode_attn(p, 1, 32, 0.1, seg, 0, out, None, p, 1 << 40, None) == SHAPE
    assert lib.kvsel_decode_attn(p, 1, 32, 0.1, seg, 5, out, None, p, 1 << 40, None) == SHAPE
    assert lib.kvsel_decode_attn(p, 1, 32, 0.1, seg, 1, None, None, p, 1 << 40, None) == NULL
    one = (K.Segment * 1)(K.Segment(FAKE, FAKE, cache(N=1300)))
    need = lib.kvsel_decode_workspace(1, 32, one, 1)
    assert need == 2 * 32 * 1 * 3 * (2 + 128) * 4          # ceil(1300 / 512) = 3 splits
    assert lib.kvsel_decode_attn(p, 1, 32, 0.1, one, 1, out, None, p, need - 4, None) == WS
    assert lib.kvsel_decode_attn(p, 1, 30, 0.1, one, 1, out, None, p, need, None) == SHAPE


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(ImportError):
        K.load(str(tmp_path / "missing.so"))


def test_gather_decode_validation(lib):
    p = ctypes.c_void_p(FAKE)
    kc = cache(B=2, N=1024, H=8, D=128)
    ext = (K.Segment * 1)(K.Segment(FAKE, FAKE, cache(B=2, N=100, H=8)))
    bad = (K.Segment * 1)(K.Segment(FAKE, FAKE, cache(B=2, N=100, H=4)))
    call = lambda k=4, unit=256, T=1, Hq=32, group=1, segs=None, n=0, idx=FAKE, ws=1 << 40, out=FAKE, vsrc=FAKE: \
        lib.kvsel_gather_decode(p, T, Hq, 0.1, p, vsrc and ctypes.c_void_p(vsrc), kc, unit,
                                idx and ctypes.c_void_p(idx), k, group, p, p, segs, n,
                                out and ctypes.c_void_p(out), None, p, ws, None)
    assert call(k=5) == SHAPE                      # M = 4
    assert call(unit=300) == SHAPE
    assert call(Hq=30) == SHAPE
    assert call(group=3) == SHAPE
    assert call(idx=0) == NULL
    assert call(vsrc=0) == NULL
    assert call(out=0) == NULL
    assert call(k=0) == SHAPE                      # nothing to attend
    assert call(n=4, segs=ext) == SHAPE            # at most 3 extra segments
    assert call(n=1, segs=None) == NULL
    assert call(n=1, segs=bad) == SHAPE            # extra segment with other H
    need = lib.kvsel_gather_decode_workspace(1, 32, kc, 256, 4, ext, 1)
    splits = (100 + 511) // 512 + (4 * 256 + 511) // 512
    assert need == 2 * 32 * 1 * splits * (2 + 128) * 4
    assert call(n=1, segs=ext, ws=need - 1) == WS
    assert lib.kvsel_gather_decode_workspace(1, 32, kc, 256, 0, None, 0) == 0


def test_score_reposition_validation(lib):
    p = ctypes.c_void_p(FAKE)
    kc = cache(B=2, N=1024, H=8, D=128)
    call = lambda rot=256, style=0, base=10000.0, delta=FAKE, kout=None, unit=256: lib.kvsel_score_reposition(
        p, 1, 32, p, kout, kc, 0.088, unit, rot, delta and ctypes.c_void_p(delta), 0, base, style,
        p, p, p, p, 1 << 40, None)
    assert call(delta=0) == NULL
    assert call(rot=300) == SHAPE
    assert call(style=3) == SHAPE
    assert call(base=1.0) == SHAPE
    assert call(kout=p) == SHAPE                  # k_out overlapping k
    assert call(kout=ctypes.c_void_p(MISALIGNED)) == UNSUP
    # streaming shape without k_out: the re-positioned keys go to the workspace
    base_ws = lib.kvsel_score_workspace(2, 1024, 32, 1, 256, 1, 1)
    need = lib.kvsel_score_reposition_workspace(1, 32, kc, 256, 256, 1, 1, 0)
    assert need == (base_ws + 255) // 256 * 256 + 2 * 1024 * 8 * 128 * 2
    assert lib.kvsel_score_reposition_workspace(1, 32, kc, 256, 256, 1, 1, 1) == base_ws
    # matrix-core shape (32 rows per kv head): fused, no extra room
    assert lib.kvsel_score_reposition_workspace(32, 32, kc, 256, 256, 1, 1, 0) == \
        lib.kvsel_score_workspace(2, 1024, 32, 32, 256, 1, 1)
