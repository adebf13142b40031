"""Pins for the phase-coherent (PCT) attention oracle (CPU only).

Hand-derived scores and outputs, the bound |s| <= sqrt(d_h) with its
equality cases, scale invariance, phase behaviour, closed forms for q = 0
and d_h = 1, and planted mistakes that each fail at least one pin.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import pct_attention, pct_attention_rows, pct_scores

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pct_worked_examples.json")


def cplx(a):
    a = np.asarray(a, dtype=np.float64)
    return a[..., 0] + 1j * a[..., 1]


def crandn(rng, *shape):
    return (rng.standard_normal(shape) + 1j * rng.standard_normal(shape)) * np.sqrt(0.5)


def sig(x):
    return 1.0 / (1.0 + math.exp(-x))


def _expr(s):
    return float(eval(s, {"__builtins__": {}}, {"sqrt": math.sqrt}))


@pytest.mark.parametrize("bias", [0.0, -math.log(3.0), 1.5])
def test_worked_examples(bias):
    for c in json.load(open(GOLDEN))["cases"]:
        q, k, v = cplx(c["q"]), cplx(c["k"]), cplx(c["v"])
        s = np.array([[_expr(e) for e in row] for row in c["scores"]])
        np.testing.assert_allclose(pct_scores(q, k), s, rtol=0, atol=1e-14, err_msg=c["name"])
        T = len(q)
        for causal in (True, False):
            want = np.zeros_like(v)
            for i in range(T):
                for j in range(i + 1 if causal else T):
                    want[i] += sig(s[i, j] + bias) * v[j]
            np.testing.assert_allclose(pct_attention(q, k, v, causal=causal, bias=bias), want, atol=1e-14)


def test_score_bound_and_equality_cases():
    rng = np.random.default_rng(1)
    for d in (1, 2, 16, 64):
        q, k = crandn(rng, 200, d), crandn(rng, 200, d)
        s = pct_scores(q, k)
        assert np.abs(s).max() <= math.sqrt(d) * (1 + 1e-12)
        # q_i parallel to k_j with a positive factor: s = +sqrt(d); anti-parallel: -sqrt(d)
        kk = np.stack([q[0] * 3.0, -q[0] * 0.2])
        s2 = pct_scores(q[:1], kk)
        np.testing.assert_allclose(s2[0], [math.sqrt(d), -math.sqrt(d)], rtol=1e-12)
    # for d = 64, b = 0, a key equal to its query gets weight sigmoid(8) = 0.99966465...
    q = crandn(rng, 1, 64)
    O = pct_attention(q, q, np.ones((1, 64)), causal=True)
    np.testing.assert_allclose(O.real, 1.0 / (1.0 + math.exp(-8.0)), rtol=1e-13)


def test_scale_invariance_per_token():
    rng = np.random.default_rng(2)
    T, d = 45, 8
    q, k, v = crandn(rng, T, d), crandn(rng, T, d), crandn(rng, T, d)
    lam = np.exp(rng.uniform(np.log(1e-3), np.log(1e3), T))
    mu = np.exp(rng.uniform(np.log(1e-3), np.log(1e3), T))
    for causal in (True, False):
        base = pct_attention(q, k, v, causal=causal)
        np.testing.assert_allclose(pct_attention(lam[:, None] * q, mu[:, None] * k, v, causal=causal), base,
                                   rtol=1e-12, atol=1e-13)


def test_phase_behaviour():
    rng = np.random.default_rng(3)
    T, d = 30, 8
    q, k, v = crandn(rng, T, d), crandn(rng, T, d), crandn(rng, T, d)
    base = pct_attention(q, k, v, causal=True)
    g = np.exp(0.77j)
    # a common global phase on q and k, or conjugating both, leaves Re<q,k> unchanged
    np.testing.assert_allclose(pct_attention(g * q, g * k, v, causal=True), base, rtol=1e-12)
    np.testing.assert_allclose(pct_attention(q.conj(), k.conj(), v, causal=True), base, rtol=1e-12)
    # a phase on q alone rotates <q,k> and changes its real part
    assert np.abs(pct_attention(g * q, k, v, causal=True) - base).max() > 1e-2


def test_zero_query_closed_form():
    rng = np.random.default_rng(4)
    T, d = 21, 4
    k, v = crandn(rng, T, d), crandn(rng, T, d)
    q = np.zeros((T, d), dtype=np.complex128)
    for b in (0.0, -math.log(T)):
        np.testing.assert_allclose(pct_attention(q, k, v, causal=True, bias=b), sig(b) * np.cumsum(v, 0), rtol=1e-13)
        np.testing.assert_allclose(pct_attention(q, k, v, causal=False, bias=b),
                                   np.broadcast_to(sig(b) * v.sum(0), (T, d)), rtol=1e-13)
    # zero keys behave the same way
    np.testing.assert_allclose(pct_attention(k, np.zeros_like(k), v, causal=True), 0.5 * np.cumsum(v, 0), rtol=1e-13)


def test_d1_score_is_cosine_of_phase_difference():
    rng = np.random.default_rng(5)
    T = 25
    a, b = rng.uniform(-np.pi, np.pi, T), rng.uniform(-np.pi, np.pi, T)
    q = (rng.uniform(0.1, 5, T) * np.exp(1j * a))[:, None]
    k = (rng.uniform(0.1, 5, T) * np.exp(1j * b))[:, None]
    np.testing.assert_allclose(pct_scores(q, k), np.cos(a[:, None] - b[None, :]), atol=1e-14)


def test_real_inputs_give_cosine_similarity():
    rng = np.random.default_rng(6)
    d = 16
    q, k = rng.standard_normal((10, d)), rng.standard_normal((12, d))
    cos = (q / np.linalg.norm(q, axis=1, keepdims=True)) @ (k / np.linalg.norm(k, axis=1, keepdims=True)).T
    np.testing.assert_allclose(pct_scores(q.astype(complex), k.astype(complex)), 4.0 * cos, rtol=1e-12)
    from sklearn.metrics.pairwise import cosine_similarity
    np.testing.assert_allclose(pct_scores(q.astype(complex), k.astype(complex)), 4.0 * cosine_similarity(q, k),
                               rtol=1e-12, atol=1e-14)


def test_rows_match_full():
    rng = np.random.default_rng(7)
    B, H, T, d = 2, 2, 31, 8
    q, k, v = crandn(rng, B, H, T, d), crandn(rng, B, H, T, d), crandn(rng, B, H, T, d)
    rows = np.array([[b, h, t] for b in range(B) for h in range(H) for t in (0, 5, T - 1)])
    for causal in (True, False):
        full = pct_attention(q, k, v, causal=causal, bias=-0.5)
        got = pct_attention_rows(q, k, v, rows, causal=causal, bias=-0.5)
        np.testing.assert_allclose(got, full[rows[:, 0], rows[:, 1], rows[:, 2]], rtol=1e-12, atol=1e-14)


def _mutants():
    def unit(x):
        return x / np.linalg.norm(x, axis=-1, keepdims=True)

    def gate(s, v, causal, b):
        w = 1 / (1 + np.exp(-(s + b)))
        if causal:
            w = w * np.tril(np.ones(w.shape))
        return w @ v

    def no_conj(q, k, v, causal=False, bias=0.0):
        return gate(math.sqrt(q.shape[-1]) * (unit(q) @ unit(k).T).real, v, causal, bias)

    def no_scale(q, k, v, causal=False, bias=0.0):
        return gate((unit(q) @ unit(k).conj().T).real, v, causal, bias)

    def no_norm(q, k, v, causal=False, bias=0.0):
        return gate(math.sqrt(q.shape[-1]) * (q @ k.conj().T).real, v, causal, bias)

    def imag_part(q, k, v, causal=False, bias=0.0):
        return gate(math.sqrt(q.shape[-1]) * (unit(q) @ unit(k).conj().T).imag, v, causal, bias)

    def row_normalised(q, k, v, causal=False, bias=0.0):
        w = 1 / (1 + np.exp(-(math.sqrt(q.shape[-1]) * (unit(q) @ unit(k).conj().T).real + bias)))
        return (w / w.sum(1, keepdims=True)) @ v

    return [no_conj, no_scale, no_norm, imag_part, row_normalised]


@pytest.mark.parametrize("mutant", _mutants(), ids=lambda f: f.__name__)
def test_planted_mistakes_fail_a_pin(mutant):
    failures = 0
    for c in json.load(open(GOLDEN))["cases"]:
        q, k, v = cplx(c["q"]), cplx(c["k"]), cplx(c["v"])
        T = len(q)
        s = np.array([[_expr(e) for e in row] for row in c["scores"]])
        want = np.array([sum(sig(s[i, j]) * v[j] for j in range(T)) for i in range(T)])
        if not np.allclose(mutant(q, k, v, causal=False), want, atol=1e-12):
            failures += 1
    assert failures > 0
