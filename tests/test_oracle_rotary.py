"""Pins for the rotary oracle (CPU only): modulus preserved, identity at
position 0, step-mode consistency (a token rotated alone at its absolute
position), additive composition for one token, channel 0 turns by exactly one
radian per position, a hand-worked value, and the property that makes it a
relative position code for Born attention -- shifting every position by the
same amount leaves |<R q_t, R k_j>|^2 unchanged (*Show HN: CNET*, the
RotaryEmbed layer: position enters as a phase rotation)."""
import math

import numpy as np

from oracle import born_attention, rotary


def crandn(rng, *shape):
    return (rng.standard_normal(shape) + 1j * rng.standard_normal(shape)) * np.sqrt(0.5)


def test_modulus_identity_and_composition():
    rng = np.random.default_rng(51)
    x = crandn(rng, 3, 40, 16)
    np.testing.assert_allclose(np.abs(rotary(x, pos0=123)), np.abs(x), rtol=1e-13)
    np.testing.assert_allclose(rotary(x[..., :1, :], pos0=0), x[..., :1, :], rtol=0, atol=0)
    # step mode: token t rotated alone at absolute position p + t is row t of the sequence rotated from p
    full = rotary(x, pos0=7)
    for t in (0, 1, 17, 39):
        np.testing.assert_allclose(rotary(x[..., t:t + 1, :], pos0=7 + t)[..., 0, :], full[..., t, :], rtol=1e-13)
    # one token: positions compose additively
    one = x[..., :1, :]
    np.testing.assert_allclose(rotary(rotary(one, pos0=7), pos0=5), rotary(one, pos0=12), rtol=1e-12, atol=1e-13)


def test_channel_frequencies():
    T, d = 10, 8
    x = np.ones((T, d), dtype=complex)
    y = rotary(x, pos0=3, base=10000.0)
    # channel 0: theta = 1, angle = position
    np.testing.assert_allclose(np.angle(y[:, 0]), np.angle(np.exp(1j * (3 + np.arange(T)))), atol=1e-13)
    # channel m: theta = 10000^(-m/d); hand value for m = 4, t = 2 (position 5): 5 * 10000^-0.5 = 0.05
    np.testing.assert_allclose(y[2, 4], np.exp(1j * 0.05), rtol=1e-14)
    # a different base changes every channel but the first
    z = rotary(x, pos0=3, base=500.0)
    np.testing.assert_allclose(z[:, 0], y[:, 0], rtol=1e-14)
    assert np.abs(z[:, 1:] - y[:, 1:]).max() > 1e-3


def test_relative_position_for_born():
    rng = np.random.default_rng(52)
    T, d = 24, 8
    q, k, v = crandn(rng, T, d), crandn(rng, T, d), crandn(rng, T, d)
    base = born_attention(rotary(q, pos0=0), rotary(k, pos0=0), v, causal=True)
    shifted = born_attention(rotary(q, pos0=1000), rotary(k, pos0=1000), v, causal=True)
    np.testing.assert_allclose(shifted, base, rtol=1e-9, atol=1e-12)
    # a shift of the keys alone is not a relative change: the output moves
    moved = born_attention(rotary(q, pos0=0), rotary(k, pos0=3), v, causal=True)
    assert np.abs(moved - base).max() > 1e-3
