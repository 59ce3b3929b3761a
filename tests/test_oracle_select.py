"""Pins of the oracle's top-k, gather/refill and the methods' host arithmetic."""

import itertools
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
from conftest import read_golden

RNG = np.random.default_rng(7)


# --- arg-top-k ([ACRE Eq. 16]) -------------------------------------------------

def _dominant_subset(s, k):
    """Brute force: the unique k-subset whose every member beats every
    non-member under (score desc, index asc)."""
    M = len(s)
    beats = lambda a, b: s[a] > s[b] or (s[a] == s[b] and a < b)
    found = [S for S in itertools.combinations(range(M), k)
             if all(beats(a, b) for a in S for b in set(range(M)) - set(S))]
    assert len(found) == 1
    return list(found[0])


@pytest.mark.parametrize("M", [1, 4, 7, 9])
def test_topk_brute_force_with_ties(M):
    for trial in range(20):
        s = RNG.integers(0, 4, size=M).astype(np.float64)      # many ties
        for k in range(0, M + 1):
            got = O.topk(s[None], k)[0].tolist()
            assert got == _dominant_subset(s, k)


def test_topk_ascending_output_and_edges():
    s = RNG.random((3, 50))
    idx = O.topk(s, 10)
    assert (np.diff(idx, axis=1) > 0).all()
    assert O.topk(s, 0).shape == (3, 0)
    assert np.array_equal(O.topk(s, 50), np.tile(np.arange(50), (3, 1)))


def test_topk_all_tied_takes_lowest_indices():
    # q = 0 makes every attention weight equal -> all scores tie
    q = np.zeros((1, 2, 2, 8))
    s = O.aggregate(q, RNG.standard_normal((1, 40, 2, 8)), None, 0.3, "mass", 4)
    assert np.array_equal(O.topk(s, 3)[0], [0, 1, 2])


def test_topk_negative_zero_ties_positive_zero():
    s = np.array([[0.0, -0.0, 0.0, 1.0]])
    assert O.topk(s, 2)[0].tolist() == [0, 3]


# --- gather and the refill layout ([ACRE Eq. 18-19]) ----------------------------

def test_refill_layout_worked_example():
    g = read_golden("acre_refill_eq18_19.txt")
    m, l = int(g["m"]), int(g["l"])
    sel0 = int(g["selected_1based"]) - 1
    # label rows: L1 entry j -> 1000 + j (1-based), L2 row i -> i (1-based)
    l1 = np.array([1000 + j for j in range(1, m + 1)], dtype=np.float64)
    l2 = np.array([i for i in range(1, m * l + 1)], dtype=np.float64)
    got = O.refill_nested(l1, l2, [sel0], l)
    names = [f"L1:{int(x) - 1000}" if x >= 1000 else f"L2:{int(x)}" for x in got]
    assert names == g["layout"].split()


def test_refill_layout_general():
    m, l = 6, 4
    l1 = np.arange(m) + 100.0
    l2 = np.arange(m * l, dtype=np.float64)
    out = O.refill_nested(l1, l2, [0, 3, 5], l)
    assert out.tolist() == [0, 1, 2, 3, 100, 101, 102, 12, 13, 14, 15, 103, 104,
                            20, 21, 22, 23, 105]


def test_gather_copies_kept_units_in_order():
    k = RNG.standard_normal((2, 24, 2, 4))
    v = RNG.standard_normal((2, 24, 2, 4))
    idx = np.array([[1, 4], [0, 5]])
    gk, gv = O.gather(k, v, idx, 4)
    assert np.array_equal(gk[0], np.concatenate([k[0, 4:8], k[0, 16:20]]))
    assert np.array_equal(gv[1], np.concatenate([v[1, 0:4], v[1, 20:24]]))
    # keeping every unit is the identity
    allk, allv = O.gather(k, v, np.tile(np.arange(6), (2, 1)), 4)
    assert np.array_equal(allk, k) and np.array_equal(allv, v)
    # one index row shared by a group of instances
    gk2, _ = O.gather(k, v, idx[:1], 4, idx_group=2)
    assert np.array_equal(gk2[1], np.concatenate([k[1, 4:8], k[1, 16:20]]))


def test_gather_aligned_is_reposition_to_contiguous_slots():
    U, n = 8, 5
    k = O.round_bf16(RNG.standard_normal((1, U * n, 2, 16)))
    p_old = np.tile(np.arange(U), n)[None]
    idx = np.array([[1, 2, 4]])
    got = O.gather_aligned(k, idx, U, p_old, align_base=64)
    for r, u in enumerate(idx[0]):
        rows = slice(u * U, (u + 1) * U)
        want = O.reposition(k[0, rows], p_old[0, rows], 64 + r * U + np.arange(U))
        assert np.array_equal(got[0, r * U:(r + 1) * U], want)
    # relative property: the dot product of a query at position P with the kept
    # key at slot r equals that of the query at P - (64 + r*U) with the stored key
    q = RNG.standard_normal(16)
    P = 500.0
    r, u, t = 1, 2, 3
    lhs = O.rope_rotate(q, P) @ got[0, r * U + t, 0]
    rhs = O.rope_rotate(q, P - (64 + r * U)) @ k[0, u * U + t, 0]
    assert lhs == pytest.approx(rhs, abs=2e-2 * np.linalg.norm(q) * np.linalg.norm(k[0, u * U + t, 0]) / 8)


# --- host arithmetic of the three methods -------------------------------------

def test_acre_eq17_k():
    # [ACRE Eq. 17] k = floor(min(W - m, eta) / l) with the main-run constants
    # l = 16, eta = 4096, W = 32K ([ACRE App. A]) ...
    W, eta, l = 32768, 4096, 16
    assert O.acre_k(W, 131072 // l, eta, l) == 256           # 128K context, m = 8192
    assert O.acre_k(W, 65536 // l, eta, l) == 256
    assert O.acre_k(W, 1048576 // l, eta, l) == 0            # m > W: clamped
    assert O.acre_k(W, 32768, eta, l) == 0                   # m == W
    assert O.acre_k(W, 30000, eta, l) == (32768 - 30000) // 16
    # ... and the bi-layer workload: interval 8, 16384 L1 entries, eta >= 16384
    assert O.acre_k(32768, 16384, 16384, 8) == 2048
    assert O.acre_k(100, 10, 1000, 7) == 12


def test_cachefocus_k_prune_worked_example():
    g = read_golden("cachefocus_k_prune.txt")
    assert O.cf_k_prune(int(g["k"]), int(g["k_finish"]), int(g["L"]), int(g["n"])) == int(g["k_prune"])


def test_cachefocus_reuse_worked_examples():
    g = read_golden("cachefocus_reuse.txt")
    k, l_C, L = int(g["k"]), int(g["l_C"]), int(g["L"])
    assert O.cf_group_size(L, l_C) == int(g["windows_per_group"])
    assert O.cf_reuse_count(k, L, l_C) == int(g["N_reuse"])
    starts = O.cf_doc_starts(k, l_C, L)
    # 5 windows with continuous positions per group, groups reuse the range
    assert starts.tolist() == [0, 100, 200, 300, 400] * 4
    assert O.cf_reuse_count(int(g["qwen_k"]), int(g["qwen_L"]), int(g["qwen_l_C"])) == int(g["qwen_N_reuse"])
    qs = O.cf_doc_starts(int(g["qwen_k"]), int(g["qwen_l_C"]), int(g["qwen_L"]))
    assert len(set(qs.tolist())) == int(g["qwen_k"])        # every position unique
    # PCW places every window in parallel: a range of one window -> all start at 0
    assert O.cf_doc_starts(7, 64, 64).tolist() == [0] * 7
    assert O.cf_reuse_count(7, 64, 64) == 7


def test_cachefocus_docs_workload_positions():
    # 32 documents of 512 tokens in a 4096-position window: 8 per group, 4 reuses
    assert O.cf_reuse_count(32, 4096, 512) == 4
    assert O.cf_doc_starts(32, 512, 4096).tolist() == [512 * (u % 8) for u in range(32)]


def test_infoflow_global_positions():
    # [InfoFlow §4.2] g(t) = Delta_i + p_i(t)
    assert O.if_chunk_offsets([3, 2, 4]).tolist() == [0, 3, 5]
    assert O.if_global_positions([3, 2, 4]).tolist() == list(range(9))
    assert O.if_global_positions([1024] * 64)[1024 * 5 + 7] == 5127


def test_infoflow_budget():
    assert O.if_budget(65536) == 9830                  # 15% of 65,536 tokens
    assert O.if_budget(100) == 15
    assert O.if_budget(20) == 3
    assert O.if_budget(65536) == int(Fraction(15, 100) * 65536)
