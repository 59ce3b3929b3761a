"""Pins of the oracle's InfoFlow two-stage selection with chunk reordering (CPU).

Fixed against: hand-counted chunk fractions, hand-ordered examples (ties
included), the offsets of the already pinned ``g(t)`` (``if_chunk_offsets``)
applied to the reordered lengths (the identity order gives exactly the GLOBAL
offsets), the first stage as the plain selection on the stored keys, and the
second stage as the selection on a cache whose chunks were physically moved
into the new order.
"""

import numpy as np

from oracle import kvsel_oracle as O


def test_chunk_fractions_by_hand():
    sel = np.array([[0, 1, 2, 1024, 5000, 8191]])
    r = O.if_chunk_fractions(sel, [1024] * 8)
    want = np.zeros((1, 8))
    want[0, 0] = 3 / 1024
    want[0, 1] = 1 / 1024
    want[0, 4] = 1 / 1024
    want[0, 7] = 1 / 1024
    np.testing.assert_array_equal(r, want)
    # unequal lengths: chunk boundaries at 3, 3 + 5
    r2 = O.if_chunk_fractions(np.array([[2, 3, 7, 8]]), [3, 5, 2])
    np.testing.assert_array_equal(r2, [[1 / 3, 2 / 5, 1 / 2]])


def test_reorder_by_hand():
    r = np.array([[0.5, 0.1, 0.9, 0.1]])
    # ranked: 2 (0.9), 0 (0.5), 1 (0.1), 3 (0.1: tie, larger index after);
    # the most informative goes last, nearest the prompt
    np.testing.assert_array_equal(O.if_reorder(r), [[3, 1, 0, 2]])


def test_reordered_offsets_follow_g_of_t():
    lens = [10, 20, 30, 40]
    order = np.array([[3, 1, 0, 2]])
    delta = O.if_reordered_offsets(order, lens)
    np.testing.assert_array_equal(delta, [[60, 40, 70, 0]])
    # the same starts from the pinned g(t) offsets of the reordered lengths
    off = O.if_chunk_offsets([lens[c] for c in order[0]])
    for p, c in enumerate(order[0]):
        assert delta[0, c] == off[p]


def _request(seed, B=2, n_chunks=6, L=16, H=2, Hq=4, T=3, D=16):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, Hq, D))
    k = rng.standard_normal((B, n_chunks * L, H, D))
    v = rng.standard_normal((B, n_chunks * L, H, D))
    k[:, 2 * L:3 * L] *= 1.8                      # one informative chunk
    return q, k, v


def test_second_stage_equals_selection_on_moved_chunks():
    q, k, v = _request(1)
    lens, L, budget = [16] * 6, 16, 20
    res = O.if_two_stage(q, k, v, lens, 0.25, budget, group=2, dtype="fp64")
    order = res["order"][0]
    assert order[-1] == 2                          # the planted chunk ends nearest the prompt
    # move the chunks into the new order and select under plain GLOBAL positions
    rows = np.concatenate([np.arange(c * L, (c + 1) * L) for c in order])
    km, vm = k[:, rows], v[:, rows]
    local = np.tile(np.arange(L), 6)
    glob = O.if_global_positions(lens)
    k2 = O.reposition(km, np.broadcast_to(local, (2, 6 * L)), np.broadcast_to(glob, (2, 6 * L)),
                      dtype="fp64")
    s = O.aggregate(q, k2, vm, 0.25, "vnorm", 1, 2)
    moved = O.topk(s, budget)[0]
    np.testing.assert_array_equal(np.sort(rows[moved]), res["sel2"][0])
    np.testing.assert_allclose(s[0][np.argsort(rows)], res["score2"][0], rtol=1e-12)


def test_identity_order_gives_the_global_positions():
    # the identity order rebuilds exactly the GLOBAL offsets of the stored order
    lens = [7, 3, 12, 5]
    ident = np.arange(4)[None]
    np.testing.assert_array_equal(O.if_reordered_offsets(ident, lens)[0],
                                  O.if_chunk_offsets(lens))
    # and a reversed order puts the last chunk first
    rev = np.arange(4)[::-1][None]
    np.testing.assert_array_equal(O.if_reordered_offsets(rev, lens)[0], [20, 17, 5, 0])


def test_ties_keep_the_smaller_index_nearer_the_prompt():
    r = np.array([[0.0, 0.25, 0.0, 0.25, 1.0]])
    order = O.if_reorder(r)[0]
    assert list(order) == [2, 0, 3, 1, 4]


def test_first_stage_is_the_stored_geometry():
    q, k, v = _request(3)
    res = O.if_two_stage(q, k, v, [16] * 6, 0.25, 20, group=2, dtype="fp64")
    s = O.aggregate(q, k, v, 0.25, "vnorm", 1, 2)
    np.testing.assert_allclose(res["score1"], s, rtol=1e-12)
    np.testing.assert_array_equal(res["sel1"], O.topk(s, 20))
    assert abs(res["r"].sum() * 16 - 20) < 1e-9      # every selected token is in one chunk
