"""Pins of the oracle's CacheFocus layer-adaptive pruning (CPU only).

Each test fixes the oracle against something other than itself: the worked
pruning example of [CacheFocus App. C], a closed form for documents whose keys
are constant (the attention mass of a document is then a softmax over the
documents), invariants of the softmax, the one-layer case (which is the
single-step selection path), and re-positioning checked by rotating the
unrotated keys straight to their target positions.
"""

import numpy as np
import pytest

from oracle import kvsel_oracle as O


def test_keep_schedule_worked_example():
    # App. C: L = 28, n = 4, k = 40, k_finish = 5 -> k_prune = (40 - 5) / (28 / 4) = 5
    assert O.cf_k_prune(40, 5, 28, 4) == 5
    assert O.cf_prune_layers(28, 4) == [3, 7, 11, 15, 19, 23, 27]
    assert O.cf_keep_schedule(40, 5, 28, 4) == [35, 30, 25, 20, 15, 10, 5]


@pytest.mark.parametrize("k,k_finish,L,n", [(40, 5, 32, 5), (10, 3, 8, 2), (40, 5, 28, 3),
                                            (7, 7, 12, 4), (9, 1, 4, 4)])
def test_keep_schedule_uneven(k, k_finish, L, n):
    sched = O.cf_keep_schedule(k, k_finish, L, n)
    P = L // n
    assert len(sched) == P == len(O.cf_prune_layers(L, n))
    assert sched[-1] == k_finish
    steps = np.diff([k] + sched) * -1
    lo, hi = (k - k_finish) // P, -(-(k - k_finish) // P)
    assert set(steps.tolist()) <= {lo, hi}
    assert steps.sum() == k - k_finish


def test_prune_layers_edge_cases():
    assert O.cf_prune_layers(5, 1) == [0, 1, 2, 3, 4]
    assert O.cf_prune_layers(3, 4) == []
    assert O.cf_keep_schedule(6, 2, 3, 4) == []


def _constant_documents(c, doc_len, D=8):
    """Keys of document d at layer l all equal c[l][d] * e_3, stored at
    document-local positions.  With half-split pairs (3, 7) and rope base
    1e16, theta_3 = 1e-12: every re-positioning here turns the keys by less
    than 1e-10 rad, so q . k' = c (1 - O(1e-20)) and the logits are constant
    per document."""
    L, k = c.shape
    e = np.zeros(D)
    e[3] = 1.0
    keys = np.zeros((L, k * doc_len, 1, D))
    for l in range(L):
        for d in range(k):
            keys[l, d * doc_len:(d + 1) * doc_len, 0] = c[l, d] * e
    # stored at local positions 0..doc_len-1
    pos = np.tile(np.arange(doc_len), k)
    stored = np.stack([O.rope_rotate(keys[l], pos[:, None], 1e16, "half") for l in range(L)])
    q = np.zeros((L, 1, 1, D))
    q[:, 0, 0, 3] = 1.0
    return q, stored


def test_closed_form_constant_documents():
    # 6 documents, 4 layers, prune every 2nd layer down to 2: keep 4 then 2
    c = np.array([[0.0, 0.5, 1.0, 1.5, 2.0, 2.5],
                  [3.0, 0.0, 0.0, 0.0, 0.0, 0.0],
                  [0.0, 0.0, 0.0, 4.0, 0.0, 0.0],
                  [1.0, 2.0, 3.0, 4.0, 5.0, 6.0]])
    doc_len, scale = 4, 1.0
    q, k = _constant_documents(c, doc_len)
    res = O.cf_progressive_prune(q, k, doc_len, scale, n=2, k_finish=2, window=1 << 20,
                                 base=1e16, style="half", dtype="fp64")
    # closed form: the mass of present document d at layer l is the softmax of
    # the constants over the present documents (each row's weights sum to 1,
    # split evenly over a document's doc_len equal logits)
    ids = list(range(6))
    total = np.zeros(6)
    expect_ids, expect_tot = [], []
    for l in range(4):
        z = np.exp(scale * c[l, ids])
        total[ids] += z / z.sum()
        expect_ids.append(list(ids))
        expect_tot.append(total[ids].copy())
        keep = {1: 4, 3: 2}.get(l)
        if keep:        # largest running totals, ties to the smaller ID
            ids = sorted(sorted(ids, key=lambda d: (-total[d], d))[:keep])
    assert [list(x) for x in res["ids"]] == expect_ids
    for l in range(4):
        np.testing.assert_allclose(res["total"][l], expect_tot[l], rtol=1e-12)
    np.testing.assert_allclose(res["final_total"], total[ids], rtol=1e-12)
    assert list(res["final_align"]) == ids == [3, 5]
    # pruning by layer 3's own mass would keep [4, 5] instead: the running
    # total (document 3's large layer-2 mass) decides
    z3 = np.exp(c[3, expect_ids[3]])
    assert sorted(np.array(expect_ids[3])[np.argsort(-z3)[:2]].tolist()) == [4, 5]
    # "sort": by total, most relevant last
    assert list(res["final_sort"]) == sorted(ids, key=lambda d: (-total[d], d))[::-1]


def test_running_total_decides_not_the_pruning_layer_alone():
    # two documents; layer 0 strongly favours doc 0, layer 1 mildly favours
    # doc 1: the running total keeps doc 0, the layer-1 mass alone would not
    c = np.array([[4.0, 0.0], [0.0, 0.5]])
    q, k = _constant_documents(c, 2)
    res = O.cf_progressive_prune(q, k, 2, 1.0, n=2, k_finish=1, window=1 << 20, base=1e16,
                                 dtype="fp64")
    assert list(res["final_align"]) == [0]


def _random_request(seed, L=4, k=6, doc_len=8, Hq=4, H=2, D=16, T=3):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((L, T, Hq, D))
    kk = rng.standard_normal((L, k * doc_len, H, D))
    v = rng.standard_normal((L, k * doc_len, H, D))
    return q, kk, v


def test_mass_of_each_layer_sums_to_the_rows():
    q, k, _ = _random_request(1)
    res = O.cf_progressive_prune(q, k, 8, 0.25, n=2, k_finish=2, window=32, dtype="fp64")
    for mass in res["mass"]:
        assert abs(mass.sum() - 4 * 3) < 1e-12          # Hq * T rows, each sums to 1
    # totals are the sums of the masses of the layers a document was present in
    for l, ids in enumerate(res["ids"]):
        expect = np.zeros(len(ids))
        for j, d in enumerate(ids):
            for l2 in range(l + 1):
                where = np.flatnonzero(res["ids"][l2] == d)
                expect[j] += res["mass"][l2][where[0]]
        np.testing.assert_allclose(res["total"][l], expect, rtol=1e-12)


def test_no_pruning_keeps_every_cache():
    q, k, _ = _random_request(2)
    res = O.cf_progressive_prune(q, k, 8, 0.25, n=2, k_finish=6, window=1024, dtype="fp64")
    assert list(res["final_align"]) == list(range(6))
    np.testing.assert_allclose(res["final_total"], np.sum(res["mass"], axis=0), rtol=1e-12)
    assert sorted(res["final_sort"]) == list(range(6))


def test_one_layer_is_the_single_step_selection():
    # L = 1, n = 1: re-position the concatenation, attention mass per document,
    # keep the top k_finish -- the one-step path of the selection method
    q, k, _ = _random_request(3, L=1)
    doc_len, window = 8, 24                                   # three slots per group
    res = O.cf_progressive_prune(q, k, doc_len, 0.25, n=1, k_finish=3, window=window,
                                 dtype="bf16")
    starts = O.cf_doc_starts(6, doc_len, window)
    p_old = np.tile(np.arange(doc_len), 6)
    k_rep = O.reposition(k[0], p_old, np.repeat(starts, doc_len) + p_old, dtype="bf16")
    s = O.aggregate(q[0][None], k_rep[None], None, 0.25, "mass", doc_len)
    assert list(res["final_align"]) == list(O.topk(s, 3)[0])
    np.testing.assert_allclose(res["mass"][0], s[0], rtol=1e-12)


def test_slot_positions_with_reuse_windows():
    # window of two documents: slots 0..4 start at 0, U, 0, U, 0; keys stored
    # at local positions are re-positioned exactly as if the unrotated keys
    # were rotated straight to start_j + t
    doc_len, k_docs, D = 4, 5, 8
    rng = np.random.default_rng(4)
    k0 = rng.standard_normal((1, k_docs * doc_len, 1, D))
    local = np.tile(np.arange(doc_len), k_docs)
    stored = O.rope_rotate(k0[0], local[:, None])[None]
    q = rng.standard_normal((1, 2, 1, D))
    res = O.cf_progressive_prune(q, stored, doc_len, 0.5, n=4, k_finish=5,
                                 window=2 * doc_len, dtype="fp64")
    assert list(res["starts"][0]) == [0, 4, 0, 4, 0]
    target = np.repeat(res["starts"][0], doc_len) + local
    direct = O.rope_rotate(k0[0], target[:, None])
    A = O.attention_weights(q[0][None], direct[None], 0.5)[0]
    mass = A.reshape(1, 2, k_docs, doc_len).sum(axis=(0, 1, 3))
    np.testing.assert_allclose(res["mass"][0], mass, rtol=1e-12)


def test_final_cache_is_contiguous_and_copies_values():
    doc_len, D, L = 4, 8, 2
    rng = np.random.default_rng(5)
    k0 = rng.standard_normal((L, 5 * doc_len, 2, D))
    v = rng.standard_normal((L, 5 * doc_len, 2, D))
    local = np.tile(np.arange(doc_len), 5)
    stored = np.stack([O.rope_rotate(k0[l], local[:, None]) for l in range(L)])
    ids = np.array([3, 0, 4])
    K, V = O.cf_final_cache(stored, v, ids, doc_len, start=7, dtype="fp64")
    rows = (ids[:, None] * doc_len + np.arange(doc_len)).reshape(-1)
    for l in range(L):
        direct = O.rope_rotate(k0[l][rows], (7 + np.arange(3 * doc_len))[:, None])
        np.testing.assert_allclose(K[l], direct, atol=1e-12)
        np.testing.assert_array_equal(V[l], v[l][rows])


def test_sort_places_the_most_relevant_last():
    q, k, _ = _random_request(6, L=4, k=8)
    res = O.cf_progressive_prune(q, k, 8, 0.25, n=2, k_finish=4, window=1 << 16, dtype="fp64")
    fa, fs, tot = res["final_align"], res["final_sort"], res["final_total"]
    assert sorted(fs) == sorted(fa) and list(fa) == sorted(fa)
    by_id = dict(zip(fa.tolist(), tot.tolist()))
    seq = [by_id[d] for d in fs]
    assert seq == sorted(seq)
    assert fs[-1] == fa[int(np.argmax(tot))]


def test_layers_after_the_last_prune_only_change_the_order():
    q, k, _ = _random_request(7, L=5, k=6)                     # n = 2: prunes at 1, 3
    a = O.cf_progressive_prune(q, k, 8, 0.25, n=2, k_finish=2, window=1 << 16, dtype="fp64")
    b = O.cf_progressive_prune(q, k, 8, 0.25, n=2, k_finish=2, window=1 << 16, dtype="fp64",
                               score_after_last_prune=False)
    assert list(a["final_align"]) == list(b["final_align"])
    assert len(a["mass"]) == 5 and len(b["mass"]) == 4


def test_take_composes_index_lists():
    src = np.array([[10, 11, 12, 13], [20, 21, 22, 23]])
    idx = np.array([[3, 0], [1, 9]])
    np.testing.assert_array_equal(O.take(src, idx), [[13, 10], [21, -1]])
    # composing with the identity changes nothing; composing twice is composing the
    # composed positions
    ident = np.tile(np.arange(4), (2, 1))
    np.testing.assert_array_equal(O.take(src, ident), src)
    a = np.array([[2, 3, 1], [0, 2, 3]])
    b = np.array([[2, 0], [1, 1]])
    np.testing.assert_array_equal(O.take(O.take(src, a), b), O.take(src, O.take(a, b)))


def test_order_lists_by_score():
    rng = np.random.default_rng(8)
    s = rng.random((3, 50))
    idx = O.topk(s, 12)                                   # ascending index order
    desc = O.order(s, idx, descending=True)
    for g in range(3):
        assert sorted(desc[g]) == sorted(idx[g])
        vals = s[g, desc[g]]
        assert np.all(np.diff(vals) <= 0)
        assert desc[g, 0] == np.argmax(s[g])
        # the k largest, largest first: the same list as a full descending sort
        assert list(desc[g]) == list(np.argsort(-s[g], kind="stable")[:12])
    np.testing.assert_array_equal(O.order(s, idx, descending=False), desc[:, ::-1])


def test_order_ties_and_invalid_entries():
    s = np.array([[1.0, 2.0, 2.0, 0.0, -0.0]])
    # ties: smaller index first; -0.0 ties +0.0; repeated entries keep list order;
    # out-of-range entries come last
    idx = np.array([[4, 2, 7, 1, 3, 2]])
    np.testing.assert_array_equal(O.order(s, idx), [[1, 2, 2, 3, 4, 7]])
    np.testing.assert_array_equal(O.order(s, idx, descending=False), [[7, 4, 3, 2, 2, 1]])
