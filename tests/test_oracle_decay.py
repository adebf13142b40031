"""Pins for the decayed Born oracle (CPU only).

The reading: with a per-head gamma in (0, 1], causal Born attention weighs key
j of query k by gamma^(k - j) |<q_k, k_j>|^2, and the carried state advances
as Z <- gamma Z + k k^H (likewise M).  The oracle is checked here against what
the mathematics fixes independently of its own code:

* gamma = 1 is plain Born attention;
* d_h = 1 closed forms: with unit-modulus keys the output is a normalised
  exponential moving average of V, a geometric or arithmetico-geometric sum
  for V = z^j or V = j (with eps the query norm enters as well);
* gamma -> 0 leaves only the key at the query's own position;
* exact rational brute force over Gaussian integers with gamma = 1/2, 2/3;
* the step recursion (a second formulation) equals the quadratic form, also
  across a carried state;
* keys that are exactly zero change nothing for any row (the factor depends
  on the distance k - j only);
* the closed-form backward with decay matches finite differences;
* planted mistakes (reversed or absolute exponent, an off-by-one exponent, a
  state decayed after the token is added) fail a pin.
"""
import itertools
from fractions import Fraction as F

import numpy as np
import pytest

from oracle import born_attention, born_attention_rows, born_prefill, born_state
from oracle.born_grad import born_attention_bwd


def crandn(rng, *shape):
    return (rng.standard_normal(shape) + 1j * rng.standard_normal(shape)) * np.sqrt(0.5)


def unit_keys(rng, T):
    return np.exp(1j * rng.uniform(-np.pi, np.pi, (T, 1)))


@pytest.mark.parametrize("eps", [0.0, 0.2])
def test_gamma_one_is_plain_born(eps):
    rng = np.random.default_rng(81)
    q, k, v = crandn(rng, 2, 3, 40, 6), crandn(rng, 2, 3, 40, 6), crandn(rng, 2, 3, 40, 6)
    got, den = born_attention(q, k, v, causal=True, eps=eps, return_den=True, decay=np.ones(3))
    want, wden = born_attention(q, k, v, causal=True, eps=eps, return_den=True)
    np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(den, wden)


@pytest.mark.parametrize("gamma", [0.5, 0.9, 0.99])
def test_d1_geometric_closed_form(gamma):
    # d_h = 1, |k_j| = 1: w[k, j] = gamma^(k-j) |q_k|^2, and with V_j = z^j
    # O_k = sum_j gamma^(k-j) z^j / sum_j gamma^(k-j)
    #     = (z^(k+1) - gamma^(k+1)) / (z - gamma) * (1 - gamma) / (1 - gamma^(k+1))
    rng = np.random.default_rng(82)
    T = 30
    z = 0.8 * np.exp(0.7j)
    q, k = crandn(rng, T, 1), unit_keys(rng, T)
    v = (z ** np.arange(T))[:, None]
    kk = np.arange(T)
    want = (z ** (kk + 1) - gamma ** (kk + 1)) / (z - gamma) * (1 - gamma) / (1 - gamma ** (kk + 1))
    np.testing.assert_allclose(born_attention(q, k, v, causal=True, decay=gamma)[:, 0], want, rtol=1e-12)


@pytest.mark.parametrize("gamma,eps", [(0.5, 0.0), (0.75, 0.3), (0.97, 1.5)])
def test_d1_arithmetico_geometric_closed_form_with_eps(gamma, eps):
    # V_j = j: numerator |q_k|^2 sum_{m=0}^{k} gamma^m (k - m) = |q_k|^2 (k S0 - S1),
    # S0 = (1 - g^(k+1)) / (1 - g), S1 = g (1 - (k+1) g^k + k g^(k+1)) / (1 - g)^2,
    # denominator |q_k|^2 S0 + eps
    rng = np.random.default_rng(83)
    T = 25
    q, k = crandn(rng, T, 1), unit_keys(rng, T)
    v = np.arange(T, dtype=np.complex128)[:, None]
    g = gamma
    kk = np.arange(T)
    S0 = (1 - g ** (kk + 1)) / (1 - g)
    S1 = g * (1 - (kk + 1) * g ** kk + kk * g ** (kk + 1)) / (1 - g) ** 2
    nq = np.abs(q[:, 0]) ** 2
    want = nq * (kk * S0 - S1) / (nq * S0 + eps)
    got, den = born_attention(q, k, v, causal=True, eps=eps, return_den=True, decay=g)
    np.testing.assert_allclose(got[:, 0], want, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(den, nq * S0 + eps, rtol=1e-13)


def test_vanishing_gamma_keeps_only_the_own_position():
    rng = np.random.default_rng(84)
    q, k, v = crandn(rng, 3, 20, 5), crandn(rng, 3, 20, 5), crandn(rng, 3, 20, 5)
    got = born_attention(q, k, v, causal=True, decay=np.full(3, 1e-200))
    np.testing.assert_allclose(got, v, rtol=1e-13)


def test_exact_rationals_over_gaussian_integers():
    vals = [0, 1, -1, 1j, 1 + 1j, 2 - 1j]
    rng = np.random.default_rng(85)

    def exact(qq, kk, vv, g, eps):
        T, d = qq.shape
        out = np.zeros((T, d), complex)
        for i in range(T):
            ws = []
            for j in range(i + 1):
                s = sum(complex(qq[i][m]) * complex(kk[j][m]).conjugate() for m in range(d))
                ws.append(g ** (i - j) * (F(int(round(s.real))) ** 2 + F(int(round(s.imag))) ** 2))
            den = sum(ws) + eps
            if den == 0:
                continue
            for m in range(d):
                re = sum(w * F(int(round(vv[j][m].real))) for j, w in enumerate(ws)) / den
                im = sum(w * F(int(round(vv[j][m].imag))) for j, w in enumerate(ws)) / den
                out[i, m] = complex(float(re), float(im))
        return out

    n = 0
    for T, d in ((2, 1), (3, 1), (4, 1), (3, 2), (4, 2)):
        combos = list(itertools.product(vals, repeat=T * d))
        for _ in range(25):
            qq = np.array(combos[rng.integers(len(combos))]).reshape(T, d)
            kk = np.array(combos[rng.integers(len(combos))]).reshape(T, d)
            vv = rng.integers(-3, 4, (T, d)) + 1j * rng.integers(-3, 4, (T, d))
            for g, eps in ((F(1, 2), F(0)), (F(2, 3), F(0)), (F(1, 2), F(1, 4))):
                got = born_attention(qq, kk, vv, causal=True, eps=float(eps), decay=float(g))
                np.testing.assert_allclose(got, exact(qq, kk, vv, g, eps), rtol=0, atol=1e-13)
                n += 1
    assert n == 375


@pytest.mark.parametrize("gamma,eps", [(0.9, 0.0), (0.6, 0.25), (1.0, 0.0)])
def test_step_recursion_equals_the_quadratic_form(gamma, eps):
    rng = np.random.default_rng(86)
    T, d = 40, 4
    q, k, v = crandn(rng, T, d), crandn(rng, T, d), crandn(rng, T, d)
    out, Z, M = born_prefill(q, k, v, eps=eps, gamma=gamma)
    np.testing.assert_allclose(out, born_attention(q, k, v, causal=True, eps=eps, decay=gamma), rtol=1e-11,
                               atol=1e-13)
    # the final state is the decayed sum of outer products
    f = gamma ** (T - 1 - np.arange(T))
    np.testing.assert_allclose(Z, (k.T * f) @ k.conj(), rtol=1e-11, atol=1e-12)


def test_carried_state_splits_a_decayed_sequence():
    rng = np.random.default_rng(87)
    T, d, cut, g = 36, 3, 13, 0.85
    q, k, v = crandn(rng, T, d), crandn(rng, T, d), crandn(rng, T, d)
    Z1, M1 = born_state(k[:cut], v[:cut], gamma=g)
    out2, Z2, M2 = born_prefill(q[cut:], k[cut:], v[cut:], Z1, M1, eps=0.1, gamma=g)
    full = born_attention(q, k, v, causal=True, eps=0.1, decay=g)
    np.testing.assert_allclose(out2, full[cut:], rtol=1e-11, atol=1e-13)
    Zf, Mf = born_state(k, v, gamma=g)
    np.testing.assert_allclose(Z2, Zf, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(M2, Mf, rtol=1e-12, atol=1e-12)


def test_zero_keys_change_nothing():
    # keys that are exactly 0 carry no weight, and the factor of every other
    # key depends on the distance only: inserting zero-key tokens in front
    # shifts the outputs by that many rows and changes nothing else
    rng = np.random.default_rng(88)
    T, d, P, g = 30, 4, 7, 0.8
    q, k, v = crandn(rng, T, d), crandn(rng, T, d), crandn(rng, T, d)
    base = born_attention(q, k, v, causal=True, decay=g)
    qp = np.concatenate([crandn(rng, P, d), q])
    kp = np.concatenate([np.zeros((P, d)), k])
    vp = np.concatenate([crandn(rng, P, d), v])
    # query t + P sees the real keys at distances (t + P) - (j + P) = t - j
    np.testing.assert_allclose(born_attention(qp, kp, vp, causal=True, decay=g)[P:], base, rtol=1e-12, atol=1e-13)


def test_rows_match_full_and_per_head_gamma():
    rng = np.random.default_rng(89)
    B, H, T, d = 2, 3, 33, 5
    q, k, v = crandn(rng, B, H, T, d), crandn(rng, B, H, T, d), crandn(rng, B, H, T, d)
    gam = np.array([0.5, 0.9, 1.0])
    full = born_attention(q, k, v, causal=True, eps=0.05, decay=gam)
    rows = np.array([(b, h, t) for b in range(B) for h in range(H) for t in (0, 1, 16, 32)])
    got = born_attention_rows(q, k, v, rows, causal=True, eps=0.05, decay=gam)
    np.testing.assert_allclose(got, full[rows[:, 0], rows[:, 1], rows[:, 2]], rtol=1e-12, atol=1e-13)
    # each head takes its own gamma: head h alone with a scalar gives the same rows
    for h in range(H):
        np.testing.assert_allclose(born_attention(q[:, h], k[:, h], v[:, h], causal=True, eps=0.05, decay=gam[h]),
                                   full[:, h], rtol=1e-13, atol=1e-14)


def test_argument_checks():
    x = np.ones((4, 2), complex)
    for bad in (0.0, -0.5, 1.5, np.nan):
        with pytest.raises(ValueError):
            born_attention(x, x, x, causal=True, decay=bad)
        with pytest.raises(ValueError):
            born_state(x, x, gamma=bad)
    with pytest.raises(ValueError):
        born_attention(x, x, x, causal=False, decay=0.5)


def _fd(fwd, args, g, h=1e-6):
    out = []
    for a_idx, a in enumerate(args):
        grad = np.zeros_like(a)
        for idx in np.ndindex(a.shape):
            for unit in (1.0, 1j):
                ap, am = a.copy(), a.copy()
                ap[idx] += h * unit
                am[idx] -= h * unit
                lp = np.sum((g.conj() * fwd(*[ap if i == a_idx else x for i, x in enumerate(args)])).real)
                lm = np.sum((g.conj() * fwd(*[am if i == a_idx else x for i, x in enumerate(args)])).real)
                grad[idx] += unit * (lp - lm) / (2 * h)
        out.append(grad)
    return out


@pytest.mark.parametrize("gamma,eps", [(0.7, 0.0), (0.9, 0.3)])
def test_decayed_backward_matches_finite_differences(gamma, eps):
    rng = np.random.default_rng(90)
    T, d = 6, 3
    q, k, v, g = crandn(rng, T, d), crandn(rng, T, d), crandn(rng, T, d), crandn(rng, T, d)
    fd = _fd(lambda a, b, c: born_attention(a, b, c, causal=True, eps=eps, decay=gamma), [q, k, v], g)
    # g is the real-pair gradient of L = Re sum conj(g) O, so the closed form
    # returns real-pair gradients, which the central differences measure
    got = born_attention_bwd(q, k, v, g, causal=True, eps=eps, decay=gamma)
    for name, x, y in zip("qkv", got, fd):
        np.testing.assert_allclose(x, y, rtol=1e-6, atol=1e-8, err_msg=name)


# ----------------------------------------------------------------------------- planted mistakes

def _weights_mutant(expo):
    def f(q, k, v, g, eps):
        T = q.shape[-2]
        S = q @ k.conj().T
        kk, jj = np.meshgrid(np.arange(T), np.arange(T), indexing="ij")
        w = np.abs(S) ** 2 * np.where(jj <= kk, float(g) ** expo(kk, jj).astype(float), 0.0)
        den = w.sum(-1) + eps
        return (w @ v) / den[:, None]
    return f


def _state_after_add(q, k, v, g, eps):
    d = q.shape[-1]
    Z, M = np.zeros((d, d), complex), np.zeros((d, d, d), complex)
    out = []
    for t in range(q.shape[0]):
        rho = np.outer(k[t], k[t].conj())
        Z, M = g * (Z + rho), g * (M + v[t][:, None, None] * rho)    # decayed after adding
        out.append(np.einsum("a,cab,b->c", q[t].conj(), M, q[t]) / ((q[t].conj() @ Z @ q[t]).real + eps))
    return np.array(out)


MUTANTS = {
    "reversed_exponent": _weights_mutant(lambda kk, jj: jj - kk),
    "absolute_key_position": _weights_mutant(lambda kk, jj: jj),
    "absolute_query_position": _weights_mutant(lambda kk, jj: kk),
    "off_by_one": _weights_mutant(lambda kk, jj: kk - jj + 1),
    "state_decayed_after_add": _state_after_add,
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_fail_a_pin(name):
    mutant = MUTANTS[name]
    failures = 0
    # the d_h = 1 closed form with eps (arithmetico-geometric pin)
    rng = np.random.default_rng(91)
    T, g, eps = 25, 0.75, 0.3
    q, k = crandn(rng, T, 1), unit_keys(rng, T)
    v = np.arange(T, dtype=np.complex128)[:, None]
    kk = np.arange(T)
    S0 = (1 - g ** (kk + 1)) / (1 - g)
    S1 = g * (1 - (kk + 1) * g ** kk + kk * g ** (kk + 1)) / (1 - g) ** 2
    nq = np.abs(q[:, 0]) ** 2
    with np.errstate(all="ignore"):
        got = mutant(q, k, v, g, eps)
    if not np.allclose(got[:, 0], nq * (kk * S0 - S1) / (nq * S0 + eps), rtol=1e-9):
        failures += 1
    # the geometric pin without eps
    z = 0.8 * np.exp(0.7j)
    vz = (z ** kk)[:, None]
    with np.errstate(all="ignore"):
        got = mutant(q, k, vz, g, 0.0)
    want = (z ** (kk + 1) - g ** (kk + 1)) / (z - g) * (1 - g) / (1 - g ** (kk + 1))
    if not np.allclose(got[:, 0], want, rtol=1e-9):
        failures += 1
    assert failures > 0
