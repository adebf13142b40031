"""Pins for the PCT family's sibling gates (CPU only): the L2-softmax cell and
the screening gate core ("Complex-valued Phase-Coherent Transformers",
Appendix D.2).

The L2-softmax is checked against scipy's softmax, against the limit of the
sigmoid cell for a large negative bias (sigmoid(s + b) -> e^b e^s, so the
normalised sigmoid output tends to the softmax output), and against closed
forms; the screening gate against closed forms and a second evaluation of its
weight map.  Planted mistakes each fail one of them.
"""
import math

import numpy as np
import pytest
from scipy.special import softmax

from oracle import pct_attention, pct_scores, pct_screen_attention, pct_softmax_attention


def crandn(rng, *shape):
    return (rng.standard_normal(shape) + 1j * rng.standard_normal(shape)) * np.sqrt(0.5)


@pytest.mark.parametrize("causal", [True, False])
def test_softmax_matches_scipy(causal):
    rng = np.random.default_rng(31)
    T, d = 37, 8
    q, k, v = crandn(rng, 2, T, d), crandn(rng, 2, T, d), crandn(rng, 2, T, d)
    s = pct_scores(q, k)
    if causal:
        s = np.where(np.tril(np.ones((T, T))) > 0, s, -np.inf)
    want = softmax(s, axis=-1) @ v
    np.testing.assert_allclose(pct_softmax_attention(q, k, v, causal=causal), want, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("causal", [True, False])
def test_softmax_is_the_sigmoid_cell_at_large_negative_bias(causal):
    rng = np.random.default_rng(32)
    T, d = 29, 16
    q, k, v = crandn(rng, T, d), crandn(rng, T, d), crandn(rng, T, d)
    b = -45.0
    num = pct_attention(q, k, v, causal=causal, bias=b)
    den = pct_attention(q, k, np.ones((T, 1)), causal=causal, bias=b)
    np.testing.assert_allclose(num / den, pct_softmax_attention(q, k, v, causal=causal), rtol=1e-12, atol=1e-13)


def test_softmax_closed_forms():
    rng = np.random.default_rng(33)
    T, d = 21, 4
    q, k, v = crandn(rng, T, d), crandn(rng, T, d), crandn(rng, T, d)
    # rows sum to one: constant values come back unchanged
    c = (0.25 - 1.5j) * np.ones((T, d))
    np.testing.assert_allclose(pct_softmax_attention(q, k, c, causal=True), c, rtol=1e-13)
    # zero queries: every score is 0, uniform weights -> prefix means / the mean
    z = np.zeros((T, d), dtype=complex)
    np.testing.assert_allclose(pct_softmax_attention(z, k, v, causal=True),
                               np.cumsum(v, 0) / np.arange(1, T + 1)[:, None], rtol=1e-13)
    np.testing.assert_allclose(pct_softmax_attention(z, k, v, causal=False),
                               np.broadcast_to(v.mean(0), (T, d)), rtol=1e-13)
    # first causal row sees only its own key
    np.testing.assert_allclose(pct_softmax_attention(q, k, v, causal=True)[0], v[0], rtol=1e-13)
    # per-token positive scales on q and k leave it unchanged
    lam, mu = np.exp(rng.uniform(-5, 5, T)), np.exp(rng.uniform(-5, 5, T))
    np.testing.assert_allclose(pct_softmax_attention(lam[:, None] * q, mu[:, None] * k, v, causal=True),
                               pct_softmax_attention(q, k, v, causal=True), rtol=1e-12)


def test_screen_closed_forms():
    rng = np.random.default_rng(34)
    T, d = 23, 9
    q, k, v = crandn(rng, T, d), crandn(rng, T, d), crandn(rng, T, d)
    # a threshold at or above sqrt(d_h) gates everything off
    assert np.all(pct_screen_attention(q, k, v, causal=False, r=2.0, t=math.sqrt(d)) == 0)
    # zero queries: s = 0, w = r^2 relu(-t)^2 for every key
    z = np.zeros((T, d), dtype=complex)
    np.testing.assert_allclose(pct_screen_attention(z, k, v, causal=True, r=1.5, t=-0.4),
                               (1.5 ** 2) * 0.4 ** 2 * np.cumsum(v, 0), rtol=1e-13)
    # a threshold below every score: w = r^2 (s - t)^2, a polynomial in the score
    s = pct_scores(q, k)
    t = -math.sqrt(d) - 0.1
    want = (0.7 ** 2) * (s - t) ** 2 * np.tril(np.ones((T, T)))
    np.testing.assert_allclose(pct_screen_attention(q, k, v, causal=True, r=0.7, t=t), want @ v, rtol=1e-12)
    # hand pin, d_h = 1: s = cos(a - b); t = 0.5 keeps only |a - b| < pi / 3
    a, bb = np.array([0.0, 0.2]), np.array([0.0, 1.9])
    q1, k1 = np.exp(1j * a)[:, None], np.exp(1j * bb)[:, None]
    v1 = np.array([[1.0 + 0j], [10.0 + 0j]])
    got = pct_screen_attention(q1, k1, v1, causal=True, r=1.0, t=0.5)
    np.testing.assert_allclose(got[:, 0], [(1 - 0.5) ** 2 * 1.0, (math.cos(0.2) - 0.5) ** 2 * 1.0 + 0.0], rtol=1e-13)


def _softmax_mutants():
    def unnormalised(q, k, v, causal):
        T = q.shape[-2]
        e = np.exp(pct_scores(q, k)) * (np.tril(np.ones((T, T))) if causal else 1.0)
        return e @ v

    def mask_after_normalising(q, k, v, causal):
        T = q.shape[-2]
        w = softmax(pct_scores(q, k), axis=-1) * (np.tril(np.ones((T, T))) if causal else 1.0)
        return w @ v

    def no_sqrt_d(q, k, v, causal):
        T, d = q.shape[-2], q.shape[-1]
        e = np.exp(pct_scores(q, k) / math.sqrt(d)) * (np.tril(np.ones((T, T))) if causal else 1.0)
        return (e / e.sum(-1, keepdims=True)) @ v

    return [unnormalised, mask_after_normalising, no_sqrt_d]


@pytest.mark.parametrize("mutant", _softmax_mutants(), ids=lambda f: f.__name__)
def test_softmax_planted_mistakes_fail(mutant):
    rng = np.random.default_rng(35)
    T, d = 17, 8
    q, k, v = crandn(rng, T, d), crandn(rng, T, d), crandn(rng, T, d)
    s = pct_scores(q, k)
    want = softmax(np.where(np.tril(np.ones((T, T))) > 0, s, -np.inf), axis=-1) @ v
    assert not np.allclose(mutant(q, k, v, True), want, rtol=1e-9, atol=1e-12)
