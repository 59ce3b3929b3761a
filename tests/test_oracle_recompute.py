"""Pins of the oracle's index-based causal attention (CPU only).

Fixed against: full attention (the pinned ``decode_attention``) when every
position is the last row; a closed form when a row sees one key; brute force
with an explicit causal mask on tiny inputs; and the causal property itself
(keys after a row's position do not change it).
"""

import numpy as np

from oracle import kvsel_oracle as O


def _inputs(seed, B=2, S=5, N=12, H=2, Hq=4, D=8):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, S, Hq, D)), rng.standard_normal((B, N, H, D)),
            rng.standard_normal((B, N, H, D)))


def test_last_position_is_full_attention():
    q, k, v = _inputs(1)
    pos = np.full((2, 5), 11)
    o, lse = O.index_causal_attention(q, k, v, pos, 0.3)
    wo, wl = O.decode_attention(q, [(k, v)], 0.3)
    np.testing.assert_allclose(o, wo, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, wl, rtol=1e-12)


def test_single_key_closed_form():
    q, k, v = _inputs(2)
    pos = np.zeros((2, 5), np.int64)
    o, lse = O.index_causal_attention(q, k, v, pos, 0.3)
    for b in range(2):
        for h in range(4):
            g = h // 2
            np.testing.assert_allclose(o[b, :, h], np.broadcast_to(v[b, 0, g], (5, 8)), atol=1e-15)
            np.testing.assert_allclose(lse[b, h], 0.3 * q[b, :, h] @ k[b, 0, g], rtol=1e-12)


def test_brute_force_with_mask():
    q, k, v = _inputs(3, N=9)
    pos = np.array([[0, 3, 3, 8, 20], [2, -1, 5, 7, 1]])
    o, lse = O.index_causal_attention(q, k, v, pos, 0.5)
    for b in range(2):
        for i in range(5):
            for h in range(4):
                g = h // 2
                if pos[b, i] < 0:
                    assert np.all(o[b, i, h] == 0) and lse[b, h, i] == -np.inf
                    continue
                w = np.array([np.exp(0.5 * sum(q[b, i, h, d] * k[b, t, g, d] for d in range(8)))
                              if t <= pos[b, i] else 0.0 for t in range(9)])
                want = sum(w[t] * v[b, t, g] for t in range(9)) / w.sum()
                np.testing.assert_allclose(o[b, i, h], want, rtol=1e-10, atol=1e-12)
                np.testing.assert_allclose(lse[b, h, i], np.log(w.sum()), rtol=1e-10)


def test_keys_after_the_position_do_not_matter():
    q, k, v = _inputs(4)
    pos = np.array([[1, 4, 6, 6, 10], [0, 2, 9, 11, 3]])
    o1, l1 = O.index_causal_attention(q, k, v, pos, 0.3)
    for b in range(2):
        for i in range(5):
            # everything after row i's own position replaced: row i is unchanged
            k2, v2 = k.copy(), v.copy()
            k2[b, pos[b, i] + 1:] = 100.0
            v2[b, pos[b, i] + 1:] = -7.0
            o2, l2 = O.index_causal_attention(q, k2, v2, pos, 0.3)
            np.testing.assert_array_equal(o1[b, i], o2[b, i])
            np.testing.assert_array_equal(l1[b, :, i], l2[b, :, i])
            # and a row with a later position does see the change
            later = np.flatnonzero(pos[b] > pos[b, i])
            if later.size:
                assert not np.allclose(o1[b, later[0]], o2[b, later[0]])
