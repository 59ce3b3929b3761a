"""Pins of the oracle's rotary embedding, re-positioning and rounding.

Each test fixes the oracle to something other than itself: closed forms of the
rotation matrix, invariants the pages state, and a library's rounding.
"""

import math

import numpy as np
import pytest
import torch

import oracle as O

RNG = np.random.default_rng(1234)


# --- frequencies and pairing ------------------------------------------------

def test_theta_closed_form():
    # theta_i = base^(-2i/D): D=4 -> [1, base^-1/2]; D=8 -> powers of base^-1/4
    assert np.allclose(O.rope_theta(4, 10000.0), [1.0, 0.01], rtol=0, atol=1e-15)
    assert np.allclose(O.rope_theta(8, 10000.0), [1.0, 0.1, 0.01, 0.001], rtol=1e-14)
    assert np.allclose(O.rope_theta(2, 500000.0), [1.0])


def test_quarter_turn_direction():
    # [InfoFlow §3.2] matrix [[cos, -sin], [sin, cos]]: at angle pi/2, (1,0) -> (0,1)
    # and (0,1) -> (-1,0); the transpose turns the other way.
    p = math.pi / 2          # theta_0 = 1 for any D
    e0, e1 = np.array([1.0, 0.0]), np.array([0.0, 1.0])
    assert np.allclose(O.rope_rotate(e0, p), [0.0, 1.0], atol=1e-15)
    assert np.allclose(O.rope_rotate(e1, p), [-1.0, 0.0], atol=1e-15)
    assert np.allclose(O.rope_rotate(e0, p, transpose=True), [0.0, -1.0], atol=1e-15)


@pytest.mark.parametrize("style,partner", [("half", 2), ("interleaved", 1)])
def test_pairing(style, partner):
    # D=4: pair 0 is (0,2) split in halves, (0,1) interleaved; a quarter turn of
    # pair 0 sends e_0 to e_partner and leaves the other pair almost untouched.
    x = np.zeros(4)
    x[0] = 1.0
    y = O.rope_rotate(x, math.pi / 2, 10000.0, style)
    expect = np.zeros(4)
    expect[partner] = 1.0
    assert np.allclose(y, expect, atol=1e-15)


def test_general_angle_closed_form():
    # one pair, arbitrary angle: the 2x2 matrix written out
    D, base = 6, 10000.0
    x = RNG.standard_normal(D)
    pos = 37.0
    th = base ** (-2.0 * np.arange(3) / D)
    y = O.rope_rotate(x, pos, base, "interleaved")
    for i in range(3):
        c, s = math.cos(pos * th[i]), math.sin(pos * th[i])
        a, b = x[2 * i], x[2 * i + 1]
        assert y[2 * i] == pytest.approx(c * a - s * b, abs=1e-13)
        assert y[2 * i + 1] == pytest.approx(s * a + c * b, abs=1e-13)


# --- invariants stated on the pages -------------------------------------------

@pytest.mark.parametrize("style", ["half", "interleaved"])
def test_inverse_is_transpose(style):
    # [CacheFocus §2.3]: R^-1 = R^T, so rotating by p then by its transpose is identity
    k = RNG.standard_normal((5, 3, 64))
    p = RNG.integers(0, 70000, size=(5, 1)).astype(np.float64)
    back = O.rope_rotate(O.rope_rotate(k, p, style=style), p, style=style, transpose=True)
    assert np.abs(back - k).max() < 1e-12
    # rotating by -p undoes rotating by p
    back2 = O.rope_rotate(O.rope_rotate(k, p, style=style), -p, style=style)
    assert np.abs(back2 - k).max() < 1e-12


@pytest.mark.parametrize("style", ["half", "interleaved"])
def test_norm_and_composition(style):
    k = RNG.standard_normal((7, 2, 128))
    a = RNG.integers(0, 5000, size=(7, 1)).astype(np.float64)
    b = RNG.integers(0, 5000, size=(7, 1)).astype(np.float64)
    ra = O.rope_rotate(k, a, style=style)
    assert np.allclose(np.linalg.norm(ra, axis=-1), np.linalg.norm(k, axis=-1), rtol=1e-13)
    rab = O.rope_rotate(O.rope_rotate(k, b, style=style), a, style=style)
    assert np.abs(rab - O.rope_rotate(k, a + b, style=style)).max() < 1e-10
    assert np.array_equal(O.rope_rotate(k, 0.0, style=style), k)


@pytest.mark.parametrize("style", ["half", "interleaved"])
def test_relative_position_property(style):
    # [CacheFocus §2.1]: q_j^T k_i depends only on j - i; shifting both positions
    # by the same amount leaves the dot product unchanged.
    q0 = RNG.standard_normal(128)
    k0 = RNG.standard_normal(128)
    for (j, i, s) in [(100, 3, 4096), (5, 900, 61234), (0, 0, 17)]:
        d1 = O.rope_rotate(q0, j, style=style) @ O.rope_rotate(k0, i, style=style)
        d2 = O.rope_rotate(q0, j + s, style=style) @ O.rope_rotate(k0, i + s, style=style)
        assert d1 == pytest.approx(d2, rel=1e-9, abs=1e-9)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_reposition_two_step_equals_one_step(dtype):
    # R(p_new) R(p_old)^T k == R(p_new - p_old) k  (rotations compose by angles)
    k = O.round_to(RNG.standard_normal((4, 256, 2, 64)), dtype)
    p_old = np.tile(np.arange(64), 4 * 4).reshape(4, 256)
    delta = RNG.integers(0, 65536, size=(4, 4)).repeat(64, axis=1)
    p_new = p_old + delta
    two = O.reposition(k, p_old, p_new, dtype=dtype)
    one = O.round_to(O.rope_rotate(k, delta[..., None].astype(np.float64)), dtype)
    # both round nearly the same float64 value: equal except within float64
    # error of a rounding boundary
    assert np.mean(two == one) > 0.9999
    assert np.abs(two - one).max() <= 2.0 ** -7 * np.abs(one).max()


def test_reposition_zero_shift_is_identity():
    k = O.round_bf16(RNG.standard_normal((2, 128, 4, 128)))
    p = np.tile(np.arange(128), 2).reshape(2, 128)
    assert np.array_equal(O.reposition(k, p, p, dtype="bf16"), k)


# --- rounding to the cache dtype -----------------------------------------------

def test_round_bf16_ties_to_even():
    one = 1.0
    ulp = 2.0 ** -7
    cases = {
        one + ulp / 2: one,                     # tie -> even (1.0)
        one + 3 * ulp / 2: one + 2 * ulp,       # tie -> even (1 + 2 ulp)
        one + ulp / 2 + 2.0 ** -30: one + ulp,  # above the tie
        one + ulp / 2 - 2.0 ** -30: one,        # below the tie
        -(one + ulp / 2): -one,
        1.5 * 2.0 ** -133: 2.0 ** -132,         # subnormal tie -> even
        2.5 * 2.0 ** -133: 2.0 ** -132,
        3.39e38: (2 - 2.0 ** -7) * 2.0 ** 127,  # below the overflow tie
        3.40e38: np.inf,                        # past it
        0.0: 0.0,
    }
    got = O.round_bf16(np.array(list(cases.keys())))
    assert np.array_equal(got, np.array(list(cases.values())))


def test_round_bf16_matches_torch_on_float32_inputs():
    # for float32 inputs a direct round-to-nearest-even is what torch's
    # float32 -> bfloat16 conversion does
    x = (RNG.standard_normal(200000) * np.exp(RNG.uniform(-30, 30, 200000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.round_bf16(x.astype(np.float64)), ref)


def test_round_fp32():
    x = np.array([1.0 + 2.0 ** -24, 1.0 + 3 * 2.0 ** -24, 0.1])
    assert np.array_equal(O.round_to(x, "fp32"), [1.0, 1.0 + 2.0 ** -22, float(np.float32(0.1))])
