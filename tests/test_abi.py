"""The C ABI: library loads, exports every declared symbol, validates arguments.

CPU only: every call here fails validation before anything would be enqueued,
so no GPU is touched.  Device pointers are fake (aligned) integers.
"""

import ctypes
import os
import re

import pytest

from query_guided_kv_amd import abi as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvsel.h")

OK, NULL, SHAPE, DTYPE, UNSUP, WS = 0, -1, -2, -3, -4, -5
FAKE = 0x10000            # aligned, never dereferenced
MISALIGNED = 0x10008


@pytest.fixture(scope="module")
def lib():
    # KVSEL_TEST_LIB: another build of the same sources (the host-sanitizer
    # build runs this file against its own library)
    path = os.environ.get("KVSEL_TEST_LIB")
    if path:
        return K.load(path)
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
    assert f(cache(B=1, N=2, stride_n=1 << 24)) == UNSUP   # row stride not below 2^24
    assert b"2^24" in lib.kvsel_last_error()
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
        out and ctypes.c_void_p(out), 0, ws, wsb, None)
    assert call(sig=3) == SHAPE
    assert call(group=3) == SHAPE                  # 2 % 3 != 0
    assert call(out=0) == NULL
    assert call(rm=0) == NULL
    assert call(rm=0, rs=0) == WS                  # derives row stats: needs workspace
    assert call(part=0, rm=0, rs=0, ws=ctypes.c_void_p(FAKE), wsb=1 << 30) == NULL  # token path needs stats
    assert call(part=0, q=0, ws=ctypes.c_void_p(FAKE), wsb=1 << 30) == NULL
    # token path: per-token sums, 16 partial arrays for a small cache (B*N < 2^19)
    assert lib.kvsel_aggregate_workspace(2, 1024, 32, 1, 1, 0, 1) == 16 * 2 * 1024 * 4
    assert lib.kvsel_aggregate_workspace(8, 65536, 32, 1, 1, 0, 1) == 8 * 65536 * 4
    # chunk path: derived row stats (2 x B*Hq*T) + row-chunk sums ((ceil(B*Hq*T/64) + B) x M)
    assert lib.kvsel_aggregate_workspace(2, 1024, 32, 1, 256, 1, 0) == (2 * 2 * 32 + (1 + 2) * 4) * 4
    assert lib.kvsel_aggregate_workspace(2, 1024, 32, 1, 256, 1, 1) == (1 + 2) * 4 * 4


def test_score_units_validation(lib):
    p = ctypes.c_void_p(FAKE)
    kc = cache(B=2, N=2048, H=4, D=128)
    f = ctypes.c_void_p(FAKE)

    def call(q=FAKE, k=FAKE, unit=512, units=FAKE, n=3, delta=FAKE, style=0, base=1e4,
             rm=FAKE, rs=FAKE, part=FAKE, Hq=28, T=32, ws=None, wsb=0, c=None):
        v = lambda x: x and ctypes.c_void_p(x)
        return lib.kvsel_score_units(v(q), T, Hq, v(k), c or kc, 0.088, unit, v(units), n,
                                     v(delta), 0, base, style, v(rm), v(rs), v(part), ws, wsb,
                                     None)
    assert call(q=0) == NULL
    assert call(q=MISALIGNED) == UNSUP
    assert call(units=0) == NULL
    assert call(unit=300) == SHAPE                 # 2048 % 300 != 0
    assert call(n=0) == SHAPE
    assert call(n=1 << 22) == SHAPE                # n_units * unit_len >= 2^31
    assert call(style=5) == SHAPE
    assert call(base=1.0) == SHAPE
    # no rotation: the rope arguments are not checked, the next check fails
    assert call(delta=0, style=5, rm=0, rs=0, part=0) == NULL
    assert call(Hq=30) == SHAPE                    # not a multiple of H
    assert call(rm=0) == NULL
    assert call(rm=0, rs=0, part=0) == NULL        # nothing requested
    assert call(unit=1, rm=0, rs=0) == SHAPE       # partials need units
    # matrix-core shape (bf16, 7 * 32 rows per kv head, 512-row units): the
    # listed units are read in place, so partials alone need no workspace
    assert lib.kvsel_score_units_workspace(32, 28, kc, 512, 3, 0, 1) == 0
    # row statistics come from the partials when both are asked for; alone
    # they need one (m, s) per 256-row segment of the 3 * 512 scored rows
    assert lib.kvsel_score_units_workspace(32, 28, kc, 512, 3, 1, 1) == 0
    assert lib.kvsel_score_units_workspace(32, 28, kc, 512, 3, 1, 0) == 2 * 28 * 32 * 6 * 2 * 4
    # fp32 caches go through a copy of the listed units in the workspace tail
    k32 = cache(B=2, N=2048, H=4, D=128, dtype=K.FP32)
    need = lib.kvsel_score_units_workspace(32, 28, k32, 512, 3, 0, 1)
    assert need == 2 * 3 * 512 * 4 * 128 * 4
    assert call(c=k32) == WS
    assert call(c=k32, ws=f, wsb=need - 1) == WS
    assert lib.kvsel_score_units_workspace(32, 28, kc, 512, 0, 0, 1) == 0   # invalid sizes


def test_take_and_order_validation(lib):
    # every call below fails validation: nothing is launched
    p = ctypes.c_void_p(FAKE)
    q = ctypes.c_void_p(FAKE + 4096)
    inside = ctypes.c_void_p(FAKE + 64)           # within src's 2 x 10 int32
    assert lib.kvsel_take(p, 2, 10, q, 3, p, None) == SHAPE          # out is src
    assert lib.kvsel_take(p, 2, 10, q, 3, inside, None) == SHAPE     # out inside src
    assert lib.kvsel_take(p, 2, 10, q, 3, q, None) == SHAPE          # out is idx
    assert lib.kvsel_take(None, 2, 10, p, 3, q, None) == NULL
    assert lib.kvsel_take(p, 0, 10, p, 3, q, None) == SHAPE
    assert lib.kvsel_take(p, 2, 0, p, 3, q, None) == SHAPE
    assert lib.kvsel_take(p, 2, 10, p, -1, q, None) == SHAPE
    assert lib.kvsel_take(p, 1 << 20, 10, q, 1 << 11, ctypes.c_void_p(FAKE << 8), None) == SHAPE
    assert lib.kvsel_order(p, 1 << 23, 10, q, 3, 1, ctypes.c_void_p(FAKE << 8), None,
                           None) == SHAPE
    assert lib.kvsel_take(None, 2, 10, None, 0, None, None) == OK     # k == 0: no-op
    assert lib.kvsel_order(p, 2, 10, q, 3, 1, q, None, None) == SHAPE  # in place
    assert lib.kvsel_order(p, 2, 10, q, 3, 1, ctypes.c_void_p(FAKE + 4096 + 16), None,
                           None) == SHAPE                              # overlaps idx
    assert lib.kvsel_order(None, 2, 10, p, 3, 1, q, None, None) == NULL
    assert lib.kvsel_order(p, 2, 10, p, 3, 1, None, None, None) == NULL
    assert lib.kvsel_order(p, 2, 1 << 31, p, 3, 1, q, None, None) == SHAPE
    assert lib.kvsel_order(p, 2, 10, p, -2, 1, q, None, None) == SHAPE
    assert lib.kvsel_order(None, 2, 10, None, 0, 1, None, None, None) == OK


def test_index_attn_validation(lib):
    # every call below fails validation: nothing is launched
    p = ctypes.c_void_p(FAKE)
    kc = cache(B=2, N=4096, H=8, D=128)

    def call(q=FAKE, S=100, Hq=32, k=FAKE, v=FAKE, c=None, pos=FAKE, out=FAKE):
        z = lambda x: x and ctypes.c_void_p(x)
        return lib.kvsel_index_attn(z(q), S, Hq, 0.088, z(k), z(v), c or kc, z(pos), z(out),
                                    None, None)
    assert call(q=0) == NULL
    assert call(q=MISALIGNED) == UNSUP
    assert call(pos=0) == NULL
    assert call(out=0) == NULL
    assert call(c=cache(B=2, N=4096, H=8, D=128, dtype=K.FP32)) == UNSUP   # bf16 only
    assert call(S=0) == SHAPE
    assert call(Hq=30) == SHAPE                   # not a multiple of H
    assert call(S=1 << 27) == SHAPE               # S * Hq >= 2^31


def test_unit_fractions_and_slot_starts_validation(lib):
    # every call below fails validation: nothing is launched
    p = ctypes.c_void_p(FAKE)
    q = ctypes.c_void_p(FAKE + 4096)
    assert lib.kvsel_unit_fractions(p, 1, 10, 1024, 64, None, None) == NULL
    assert lib.kvsel_unit_fractions(None, 1, 10, 1024, 64, q, None) == NULL
    assert lib.kvsel_unit_fractions(p, 0, 10, 1024, 64, q, None) == SHAPE
    assert lib.kvsel_unit_fractions(p, 1, 10, 0, 64, q, None) == SHAPE
    assert lib.kvsel_unit_fractions(p, 1, 10, 1 << 20, 1 << 12, q, None) == SHAPE   # rows >= 2^31
    assert lib.kvsel_unit_fractions(p, 1, 10, 1024, 64, ctypes.c_void_p(FAKE + 8), None) == SHAPE
    assert lib.kvsel_slot_starts(None, 1, 64, 1024, 0, 32, q, None) == NULL
    assert lib.kvsel_slot_starts(p, 1, 64, 1024, 0, 32, None, None) == NULL
    assert lib.kvsel_slot_starts(p, 1, 64, 1024, 0, 0, q, None) == SHAPE            # rep < 1
    assert lib.kvsel_slot_starts(p, 1, 64, 1024, -1, 1, q, None) == SHAPE           # base < 0
    assert lib.kvsel_slot_starts(p, 1, 64, 1 << 25, 0, 1, q, None) == SHAPE         # positions >= 2^31
    assert lib.kvsel_slot_starts(p, 1, 64, 1024, 0, 2, ctypes.c_void_p(FAKE + 128), None) == SHAPE


def test_topk_validation(lib):
    p = ctypes.c_void_p(FAKE)
    assert lib.kvsel_topk(None, 1, 10, 2, p, None, None) == NULL
    assert lib.kvsel_topk(p, 1, 10, 11, p, None, None) == SHAPE
    assert lib.kvsel_topk(p, 1, 10, -1, p, None, None) == SHAPE
    assert lib.kvsel_topk(p, 0, 10, 1, p, None, None) == SHAPE
    assert lib.kvsel_topk(p, 1, 1 << 31, 1, p, None, None) == SHAPE
    assert lib.kvsel_topk(p, 1 << 21, 10, 1, p, None, None) == SHAPE   # grid too large
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
    wide = (K.Segment * 1)(K.Segment(FAKE, FAKE, cache(B=1, N=4, stride_n=1 << 24)))
    assert lib.kvsel_decode_attn(p, 1, 32, 0.1, wide, 1, out, None, p, 1 << 40, None) == UNSUP


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


def mfma_decode_splits(B, H, rows, n_keys):
    """Splits of a matrix-core decode: 1024 keys, halved down to 256 while the
    launch holds fewer than 2048 waves (row blocks of 16; up to 2 blocks run
    as 2 waves, up to 11 as 4 waves, 12 or more as 8 waves of 2 blocks a pass)."""
    rbs = -(-rows // 16)
    rbw, nwaves = (2, 8) if rbs >= 12 else (1, 2 if rbs <= 2 else 4)
    passes = -(-rbs // (rbw * nwaves))
    length = 1024
    while length > 256 and B * H * passes * -(-n_keys // length) * nwaves < 2048:
        length //= 2
    return length


def test_decode_split_rule():
    # small launches take shorter splits; launches that fill the chip keep 1024
    assert mfma_decode_splits(2, 4, 7, 3000) == 256
    assert mfma_decode_splits(1, 32, 32, 4096) == 256           # 32 docs x 512, 32 kv heads
    assert mfma_decode_splits(1, 4, 448, 32768) == 1024         # 448 rows: 8 waves, 2 passes
    assert mfma_decode_splits(448, 4, 7, 2560) == 1024
    assert mfma_decode_splits(1, 8, 16, 65536) == 512


def test_decode_split_by_path(lib):
    """The workspace of a decode call follows the kernel it runs: the
    streaming kernel splits the keys by 512; a plain pass with 5 or more bf16
    rows per kv head runs on the matrix cores, whose split length follows
    mfma_decode_splits; the fused refill keeps the streaming kernel (512) up
    to 8 rows."""
    N, D = 3000, 128
    seven = (K.Segment * 1)(K.Segment(FAKE, FAKE, cache(B=2, N=N, H=4, D=D)))
    # 28 / 4 heads x 1 token = 7 rows per kv head: matrix cores, a small launch
    n7 = -(-N // mfma_decode_splits(2, 4, 7, N))
    assert n7 == 12
    assert lib.kvsel_decode_workspace(1, 28, seven, 1) == 2 * 28 * 1 * n7 * (2 + D) * 4
    # 4 rows per kv head: streaming, ceil(3000 / 512) = 6 splits
    assert lib.kvsel_decode_workspace(1, 16, seven, 1) == 2 * 16 * 1 * 6 * (2 + D) * 4
    # fp32 keys: the tile kernel, 512-key splits
    f32 = (K.Segment * 1)(K.Segment(FAKE, FAKE, cache(B=2, N=N, H=4, D=D, dtype=1)))
    assert lib.kvsel_decode_workspace(1, 28, f32, 1) == 2 * 28 * 1 * 6 * (2 + D) * 4
    # the fused refill with 7 rows: streaming, the kept rows split by 512
    kc = cache(B=2, N=8 * 512, H=4, D=D)
    rows = 5 * 512
    need = lib.kvsel_gather_decode_workspace(1, 28, kc, 512, 5, None, 0)
    assert need == 2 * 28 * 1 * ((rows + 511) // 512) * (2 + D) * 4
    # with 16 rows per kv head (no streaming kernel) the copy and the plain pass
    # run separately: matrix-core splits
    need16 = lib.kvsel_gather_decode_workspace(4, 16, kc, 512, 5, None, 0)
    L16 = mfma_decode_splits(2, 4, 16, rows)
    assert need16 == 2 * 16 * 4 * -(-rows // L16) * (2 + D) * 4


def test_scale_must_be_finite_and_positive(lib):
    # every call below fails validation on its scale alone: nothing is launched
    p = ctypes.c_void_p(FAKE)
    kc = cache(B=2, N=1024, H=8, D=128)
    one = (K.Segment * 1)(K.Segment(FAKE, FAKE, kc))
    for bad in (0.0, -0.088, float("inf"), float("nan")):
        assert lib.kvsel_score(p, 1, 32, p, kc, bad, 256, p, p, p, p, 1 << 40, None) == SHAPE
        assert lib.kvsel_score_reposition(p, 1, 32, p, None, kc, bad, 256, 256, p, 0, 1e4, 0,
                                          p, p, p, p, 1 << 40, None) == SHAPE
        assert lib.kvsel_score_units(p, 32, 28, p, cache(B=2, N=2048, H=4), bad, 512, p, 3, None,
                                     0, 1e4, 0, p, p, p, p, 1 << 40, None) == SHAPE
        assert lib.kvsel_aggregate(p, 1, 32, p, p, kc, bad, p, p, p, 0, 256, 1, p, 0, p, 1 << 40,
                                   None) == SHAPE
        assert lib.kvsel_index_attn(p, 100, 32, bad, p, p, kc, p, p, None, None) == SHAPE
        assert lib.kvsel_decode_attn(p, 1, 32, bad, one, 1, p, None, p, 1 << 40, None) == SHAPE
        assert lib.kvsel_gather_decode(p, 1, 32, bad, p, p, kc, 256, p, 4, 1, p, p, None, 0, p,
                                       None, p, 1 << 40, None) == SHAPE
        assert b"scale" in lib.kvsel_last_error()


def test_launch_failure_is_reported(lib):
    """A call that passes validation but whose launch the runtime rejects
    returns KVSEL_ERR_HIP with the runtime's message.  Forced here by the
    absence of a device: on a host with a GPU the fake pointers would be
    launched on, so the case runs only where the GPU driver's device node is
    absent (no torch import: this file also runs under the host sanitizer)."""
    if os.path.exists("/dev/kfd"):
        pytest.skip("a GPU driver is present: the launch would run on fake pointers")
    p = ctypes.c_void_p(FAKE)
    assert lib.kvsel_topk(p, 1, 10, 2, p, None, None) == -6
    assert lib.kvsel_last_error().startswith(b"kvsel_topk:")
    assert lib.kvsel_take(p, 2, 10, ctypes.c_void_p(FAKE + 4096), 3,
                          ctypes.c_void_p(FAKE + 8192), None) == -6
