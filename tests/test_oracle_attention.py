"""Pins of the oracle's scoring, aggregation and final attention pass."""

import itertools

import numpy as np
import pytest
import torch

import oracle as O

RNG = np.random.default_rng(99)


def rand(*shape):
    return RNG.standard_normal(shape)


def sdpa(q, k, v):
    """torch's scaled_dot_product_attention on CPU in float64, with GQA heads
    expanded by repetition.  q [B][T][Hq][D], k/v [B][N][H][D] -> [B][T][Hq][Dv]."""
    B, T, Hq, D = q.shape
    rep = Hq // k.shape[2]
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)
    kt = torch.from_numpy(np.repeat(k, rep, axis=2)).permute(0, 2, 1, 3).contiguous()
    vt = torch.from_numpy(np.repeat(v, rep, axis=2)).permute(0, 2, 1, 3).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)
    return o.permute(0, 2, 1, 3).numpy()


# --- the softmax of [ACRE §2.1 Eq. 4] / §2.4 -----------------------------------

def test_attention_weights_match_sdpa_with_identity_values():
    # softmax(QK^T/sqrt(d)) . I_N is the attention matrix itself
    B, T, Hq, H, D, N = 2, 3, 4, 2, 16, 40
    q, k = rand(B, T, Hq, D), rand(B, N, H, D)
    eye = np.broadcast_to(np.eye(N)[None, :, None, :], (B, N, H, N)).copy()
    ref = sdpa(q, k, eye)                          # [B][T][Hq][N]
    A = O.attention_weights(q, k, 1.0 / np.sqrt(D))  # [B][Hq][T][N]
    assert np.abs(A - ref.transpose(0, 2, 1, 3)).max() < 1e-13
    assert np.allclose(A.sum(axis=-1), 1.0, atol=1e-14)


def test_logits_brute_force():
    B, T, Hq, H, D, N = 1, 2, 6, 3, 4, 5
    q, k = rand(B, T, Hq, D), rand(B, N, H, D)
    lg = O.logits(q, k, 0.5)
    for h, j, t in itertools.product(range(Hq), range(T), range(N)):
        g = h // 2
        dot = sum(q[0, j, h, d] * k[0, t, g, d] for d in range(D))
        assert lg[0, h, j, t] == pytest.approx(0.5 * dot, abs=1e-12)


def test_score_stats_and_partials():
    B, T, Hq, H, D, N, U = 2, 3, 4, 4, 8, 48, 12
    q, k = rand(B, T, Hq, D), 3 * rand(B, N, H, D)
    m, Z, part = O.score(q, k, 0.3, U)
    lg = O.logits(q, k, 0.3)
    assert np.array_equal(m, lg.max(axis=-1))
    # Z * exp(m) = sum exp(l): check against torch's logsumexp
    lse = torch.logsumexp(torch.from_numpy(lg), dim=-1).numpy()
    assert np.allclose(m + np.log(Z), lse, rtol=0, atol=1e-12)
    # partials merge back into the row statistics
    m2, Z2 = O.combine_partials(part)
    assert np.array_equal(m2, m)
    assert np.allclose(Z2, Z, rtol=1e-13)
    # each partial is the logsumexp of its unit
    lse_u = torch.logsumexp(torch.from_numpy(lg.reshape(B, Hq, T, N // U, U)), dim=-1).numpy()
    assert np.allclose(part[..., 0] + np.log(part[..., 1]), lse_u, atol=1e-12)


# --- aggregation ([ACRE Eq. 15], [CacheFocus fn. 3], [InfoFlow §4.2]) ----------

def test_mass_conservation():
    B, T, Hq, H, D, N, U, grp = 4, 5, 8, 2, 16, 64, 8, 2
    q, k, v = rand(B, T, Hq, D), rand(B, N, H, D), rand(B, N, H, D)
    s = O.aggregate(q, k, v, 0.25, "mass", U, grp)
    assert s.shape == (B // grp, N // U)
    assert np.allclose(s.sum(axis=-1), Hq * T * grp, rtol=1e-13)


def test_uniform_when_keys_equal_or_query_zero():
    B, T, Hq, H, D, N, U = 1, 4, 4, 2, 8, 96, 16
    v = rand(B, N, H, D)
    k_eq = np.broadcast_to(rand(1, 1, H, D), (B, N, H, D)).copy()
    s = O.aggregate(rand(B, T, Hq, D), k_eq, v, 0.35, "mass", U)
    assert np.allclose(s, Hq * T * U / N, rtol=1e-13)
    s0 = O.aggregate(np.zeros((B, T, Hq, D)), rand(B, N, H, D), v, 0.35, "mass", U)
    assert np.allclose(s0, Hq * T * U / N, rtol=1e-13)


def test_eq15_mean_pool_equals_scaled_sum():
    # [ACRE Eq. 15]: S = mean over heads and query tokens of A (h x m x t);
    # the summed score is the same ranking times Hq*T.
    T, Hq, D, N = 6, 4, 16, 30
    q, k, v = rand(1, T, Hq, D), rand(1, N, Hq, D), rand(1, N, Hq, D)
    A = O.attention_weights(q, k, 0.25)[0]            # [Hq][T][N]
    S_mean = O.acre_mean_pool(A.transpose(0, 2, 1))   # page order h x m x t
    S_sum = O.aggregate(q, k, v, 0.25, "mass", 1)[0]
    assert np.allclose(S_mean * Hq * T, S_sum, rtol=1e-13)


def test_token_scores_summed_per_unit_equal_chunk_scores():
    B, T, Hq, H, D, N, U = 2, 3, 4, 2, 8, 60, 6
    q, k, v = rand(B, T, Hq, D), rand(B, N, H, D), rand(B, N, H, D)
    for sig in ("mass", "vnorm"):
        tok = O.aggregate(q, k, v, 0.4, sig, 1)
        chk = O.aggregate(q, k, v, 0.4, sig, U)
        assert np.allclose(tok.reshape(B, N // U, U).sum(-1), chk, rtol=1e-13)


def test_vnorm_with_constant_norm_is_scaled_mass():
    B, T, Hq, H, D, N = 2, 3, 4, 2, 8, 50
    q, k, v = rand(B, T, Hq, D), rand(B, N, H, D), rand(B, N, H, D)
    v = 2.5 * v / np.linalg.norm(v, axis=-1, keepdims=True)
    assert np.allclose(O.aggregate(q, k, v, 0.4, "vnorm", 1),
                       2.5 * O.aggregate(q, k, v, 0.4, "mass", 1), rtol=1e-13)


def test_vnorm_brute_force():
    B, T, Hq, H, D, N = 1, 2, 4, 2, 3, 5
    q, k, v = rand(B, T, Hq, D), rand(B, N, H, D), rand(B, N, H, D)
    s = O.aggregate(q, k, v, 0.7, "vnorm", 1)[0]
    for t in range(N):
        acc = 0.0
        for h in range(Hq):
            g = h // 2
            for j in range(T):
                ls = [0.7 * sum(q[0, j, h, d] * k[0, n, g, d] for d in range(D)) for n in range(N)]
                z = sum(np.exp(x) for x in ls)
                acc += np.exp(ls[t]) / z * np.sqrt(sum(v[0, t, g, d] ** 2 for d in range(D)))
        assert s[t] == pytest.approx(acc, rel=1e-12)


@pytest.mark.parametrize("sig", ["mass", "vnorm"])
def test_gqa_equals_mha_with_replicated_heads(sig):
    B, T, Hq, H, D, N, U = 2, 3, 8, 2, 8, 40, 5
    q, k, v = rand(B, T, Hq, D), rand(B, N, H, D), rand(B, N, H, D) * np.arange(1, H + 1)[:, None]
    kr, vr = np.repeat(k, Hq // H, axis=2), np.repeat(v, Hq // H, axis=2)
    assert np.allclose(O.aggregate(q, k, v, 0.3, sig, U), O.aggregate(q, kr, vr, 0.3, sig, U), rtol=1e-13)


def test_group_sums_instances():
    B, T, Hq, H, D, N = 4, 2, 4, 4, 8, 32
    q, k, v = rand(B, T, Hq, D), rand(B, N, H, D), rand(B, N, H, D)
    one = O.aggregate(q, k, v, 0.3, "vnorm", 1, 1)
    two = O.aggregate(q, k, v, 0.3, "vnorm", 1, 2)
    assert np.allclose(two, one[0::2] + one[1::2], rtol=1e-13)


# --- final attention pass ([ACRE Eq. 4]) ----------------------------------------

def test_decode_matches_sdpa_and_logsumexp():
    B, T, Hq, H, D, N = 2, 5, 8, 2, 32, 70
    q, k, v = rand(B, T, Hq, D), rand(B, N, H, D), rand(B, N, H, D)
    o, lse = O.decode_attention(q, [(k, v)], 1.0 / np.sqrt(D))
    assert np.abs(o - sdpa(q, k, v)).max() < 1e-13
    ref = torch.logsumexp(torch.from_numpy(O.logits(q, k, 1.0 / np.sqrt(D))), dim=-1).numpy()
    assert np.allclose(lse, ref, atol=1e-12)


def test_decode_segments_equal_concatenation_and_order_free():
    B, T, Hq, H, D = 1, 3, 4, 2, 16
    q = rand(B, T, Hq, D)
    k1, v1, k2, v2 = rand(B, 20, H, D), rand(B, 20, H, D), rand(B, 9, H, D), rand(B, 9, H, D)
    o2, l2 = O.decode_attention(q, [(k1, v1), (k2, v2)], 0.25)
    K, V = np.concatenate([k1, k2], 1), np.concatenate([v1, v2], 1)
    perm = RNG.permutation(29)
    o1, l1 = O.decode_attention(q, [(K[:, perm], V[:, perm])], 0.25)
    assert np.abs(o2 - o1).max() < 1e-13 and np.abs(l2 - l1).max() < 1e-13


def test_decode_single_key_returns_its_value():
    q, k, v = rand(1, 2, 4, 8), rand(1, 1, 4, 8), rand(1, 1, 4, 8)
    o, lse = O.decode_attention(q, [(k, v)], 0.5)
    assert np.allclose(o, np.broadcast_to(v[:, 0][:, None], o.shape), atol=1e-15)
