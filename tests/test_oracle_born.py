"""Pins for the Born-rule attention oracle (CPU only).

The oracle (plain fp64 definition) is checked here against things other than
itself: hand-derived worked examples, closed forms, invariants the definition
implies, and a second formulation through density-matrix prefix states.  A
planted-mistake test at the end shows that plausible slips (a dropped
conjugate, transposed operands, a dropped square, an exclusive mask) fail
at least one pin.
"""
import json
import os

import numpy as np
import pytest

from oracle import born_attention, born_attention_rows, born_attention_density

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "born_worked_examples.json")


def cplx(a):
    a = np.asarray(a, dtype=np.float64)
    return a[..., 0] + 1j * a[..., 1]


def crandn(rng, *shape):
    return (rng.standard_normal(shape) + 1j * rng.standard_normal(shape)) * np.sqrt(0.5)


def test_worked_examples():
    cases = json.load(open(GOLDEN))["cases"]
    assert len(cases) >= 3
    for c in cases:
        q, k, v = cplx(c["q"]), cplx(c["k"]), cplx(c["v"])
        for mode, causal in (("causal", True), ("full", False)):
            want = cplx(c[mode]["O"])
            got = born_attention(q, k, v, causal=causal)
            np.testing.assert_allclose(got, want, rtol=0, atol=1e-14, err_msg=f"{c['name']} {mode}")


def test_rows_sum_to_one_constant_v():
    # a constant value vector c in every position must come back unchanged: the weights are a distribution
    rng = np.random.default_rng(1)
    for causal in (True, False):
        q, k = crandn(rng, 3, 37, 8), crandn(rng, 3, 37, 8)
        c = crandn(rng, 8)
        v = np.broadcast_to(c, (3, 37, 8))
        np.testing.assert_allclose(born_attention(q, k, v, causal=causal), np.broadcast_to(c, (3, 37, 8)), atol=1e-13)


def test_one_hot_values_expose_weight_matrix():
    rng = np.random.default_rng(2)
    T = 16
    q, k = crandn(rng, T, T), crandn(rng, T, T)
    v = np.eye(T, dtype=np.complex128)            # V_j = e_j  =>  O_k = A_k,:
    A = born_attention(q, k, v, causal=True)
    assert np.abs(A.imag).max() < 1e-15
    A = A.real
    assert A.min() >= 0.0
    assert np.abs(np.triu(A, 1)).max() == 0.0     # no weight on future keys
    np.testing.assert_allclose(A.sum(1), 1.0, atol=1e-14)
    assert A[0, 0] == pytest.approx(1.0, abs=1e-15)
    # the weights are |<q_k,k_j>|^2 up to the row scale: ratios are fixed by two entries
    S = np.abs(np.array([[np.vdot(k[j], q[i]) for j in range(T)] for i in range(T)])) ** 2
    i = T - 1
    np.testing.assert_allclose(A[i, :] / A[i, 0], S[i, :] / S[i, 0], rtol=1e-10)


def test_first_causal_row_returns_v0():
    rng = np.random.default_rng(3)
    q, k, v = crandn(rng, 2, 5, 64, 16), crandn(rng, 2, 5, 64, 16), crandn(rng, 2, 5, 64, 16)
    O = born_attention(q, k, v, causal=True)
    np.testing.assert_allclose(O[..., 0, :], v[..., 0, :], atol=1e-14)


def test_per_token_phase_and_scale_invariance():
    rng = np.random.default_rng(4)
    T, d = 50, 8
    q, k, v = crandn(rng, T, d), crandn(rng, T, d), crandn(rng, T, d)
    base = born_attention(q, k, v, causal=True)
    # q_k -> c_k q_k for any nonzero complex c_k (phase and modulus), k_j -> e^{i psi_j} k_j, K -> c K
    cq = rng.uniform(0.01, 100, T) * np.exp(1j * rng.uniform(0, 2 * np.pi, T))
    pk = np.exp(1j * rng.uniform(0, 2 * np.pi, T))
    np.testing.assert_allclose(born_attention(cq[:, None] * q, pk[:, None] * k, v), base, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(born_attention(q, (3.7 - 2.1j) * k, v), base, rtol=1e-10, atol=1e-12)
    # a global phase on Q or on K (the weaker statement)
    np.testing.assert_allclose(born_attention(np.exp(0.3j) * q, k, v), base, rtol=1e-12, atol=1e-13)
    # but a per-component (non-global) phase on K does change the output
    other = born_attention(q, k * np.exp(1j * np.arange(d))[None, :], v)
    assert np.abs(other - base).max() > 1e-3


def test_d1_closed_form_cumulative_weighted_mean():
    # d_h = 1: |q_k conj(k_j)|^2 = |q_k|^2 |k_j|^2, so O_k = sum_{j<=k} |k_j|^2 v_j / sum_{j<=k} |k_j|^2
    rng = np.random.default_rng(5)
    T = 40
    q, k, v = crandn(rng, T, 1), crandn(rng, T, 1), crandn(rng, T, 1)
    wk = np.abs(k[:, 0]) ** 2
    want = np.cumsum(wk * v[:, 0]) / np.cumsum(wk)
    np.testing.assert_allclose(born_attention(q, k, v, causal=True)[:, 0], want, rtol=1e-12)
    want_full = np.sum(wk * v[:, 0]) / np.sum(wk)
    np.testing.assert_allclose(born_attention(q, k, v, causal=False)[:, 0], want_full, rtol=1e-12)


def test_equal_keys_give_prefix_mean():
    rng = np.random.default_rng(6)
    T, d = 33, 4
    q, v = crandn(rng, T, d), crandn(rng, T, d)
    k = np.broadcast_to(crandn(rng, d), (T, d))
    want = np.cumsum(v, axis=0) / np.arange(1, T + 1)[:, None]
    np.testing.assert_allclose(born_attention(q, k, v, causal=True), want, rtol=1e-12)
    np.testing.assert_allclose(born_attention(q, k, v, causal=False), np.broadcast_to(v.mean(0), (T, d)), rtol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("T,d", [(1, 1), (7, 3), (24, 8), (40, 16)])
def test_density_matrix_formulation_agrees(causal, T, d):
    rng = np.random.default_rng(100 + T + d)
    q, k, v = crandn(rng, T, d), crandn(rng, T, d), crandn(rng, T, d)
    np.testing.assert_allclose(born_attention(q, k, v, causal=causal),
                               born_attention_density(q, k, v, causal=causal), rtol=1e-10, atol=1e-12)


def test_eps_and_zero_denominator():
    rng = np.random.default_rng(7)
    T, d = 9, 4
    q, k = crandn(rng, T, d), crandn(rng, T, d)
    c = crandn(rng, d)
    v = np.broadcast_to(c, (T, d))
    eps = 0.25
    O, den = born_attention(q, k, v, causal=True, eps=eps, return_den=True)
    S = np.abs(np.conj(k) @ q.T).T ** 2                 # S[i, j] = |<q_i,k_j>|^2
    tot = np.array([S[i, : i + 1].sum() for i in range(T)])
    np.testing.assert_allclose(den, tot + eps, rtol=1e-12)
    np.testing.assert_allclose(O, (tot / (tot + eps))[:, None] * c[None, :], rtol=1e-12)
    # keys all zero: every weight is 0, the denominator is 0, the output is 0
    Oz = born_attention(q, np.zeros_like(k), v, causal=True)
    assert np.all(Oz == 0)


def test_rows_match_full():
    rng = np.random.default_rng(8)
    B, H, T, d = 2, 3, 29, 8
    q, k, v = crandn(rng, B, H, T, d), crandn(rng, B, H, T, d), crandn(rng, B, H, T, d)
    rows = np.array([[b, h, t] for b in range(B) for h in range(H) for t in (0, 1, 13, T - 1)])
    for causal in (True, False):
        full = born_attention(q, k, v, causal=causal)
        got = born_attention_rows(q, k, v, rows, causal=causal)
        np.testing.assert_allclose(got, full[rows[:, 0], rows[:, 1], rows[:, 2]], rtol=1e-12, atol=1e-14)


def test_heads_are_independent():
    rng = np.random.default_rng(9)
    B, H, T, d = 2, 3, 17, 4
    q, k, v = crandn(rng, B, H, T, d), crandn(rng, B, H, T, d), crandn(rng, B, H, T, d)
    full = born_attention(q, k, v)
    for b in range(B):
        for h in range(H):
            np.testing.assert_allclose(full[b, h], born_attention(q[b, h], k[b, h], v[b, h]), rtol=1e-13)


def test_exhaustive_small_gaussian_integers():
    # brute force with exact rational arithmetic over Gaussian integers: T <= 3, d_h = 1 and 2
    from fractions import Fraction as F
    import itertools
    vals = [0, 1, -1, 1j, 1 + 1j]
    rng = np.random.default_rng(10)

    def exact(qq, kk, vv, causal):
        T = len(qq)
        out = []
        for i in range(T):
            J = range(i + 1) if causal else range(T)
            ws = []
            for j in J:
                s = sum(complex(qq[i][m]) * complex(kk[j][m]).conjugate() for m in range(len(qq[i])))
                ws.append(F(int(round(s.real))) ** 2 + F(int(round(s.imag))) ** 2)
            den = sum(ws)
            row = []
            for m in range(len(vv[0])):
                if den == 0:
                    row.append(0j)
                    continue
                re = sum(w * F(int(round(vv[j][m].real))) for w, j in zip(ws, J)) / den
                im = sum(w * F(int(round(vv[j][m].imag))) for w, j in zip(ws, J)) / den
                row.append(complex(float(re), float(im)))
            out.append(row)
        return np.array(out)

    n = 0
    for T, d in ((1, 1), (2, 1), (3, 1), (2, 2), (3, 2)):
        combos = list(itertools.product(vals, repeat=T * d))
        for _ in range(60):
            qq = np.array(combos[rng.integers(len(combos))]).reshape(T, d)
            kk = np.array(combos[rng.integers(len(combos))]).reshape(T, d)
            vv = (rng.integers(-3, 4, (T, d)) + 1j * rng.integers(-3, 4, (T, d)))
            for causal in (True, False):
                np.testing.assert_allclose(born_attention(qq, kk, vv, causal=causal), exact(qq, kk, vv, causal),
                                           rtol=0, atol=1e-13)
                n += 1
    assert n == 600


def test_real_inputs_match_library_polynomial_kernel():
    # real Q, K: |<q,k>|^2 is the degree-2 homogeneous polynomial kernel (q.k)^2 of scikit-learn
    from sklearn.metrics.pairwise import polynomial_kernel
    rng = np.random.default_rng(12)
    T, d = 20, 6
    q, k = rng.standard_normal((T, d)), rng.standard_normal((T, d))
    v = crandn(rng, T, d)
    s = polynomial_kernel(q, k, degree=2, gamma=1.0, coef0=0.0)
    for causal in (True, False):
        w = np.tril(s) if causal else s
        want = (w @ v) / w.sum(1, keepdims=True)
        np.testing.assert_allclose(born_attention(q.astype(complex), k.astype(complex), v, causal=causal), want,
                                   rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------------------- planted mistakes

def _mutants():
    def no_conj(q, k, v, causal=True, eps=0.0):
        T = q.shape[-2]
        S = q @ np.swapaxes(k, -1, -2)
        s = np.abs(S) ** 2
        s = s * np.tril(np.ones((T, T))) if causal else s
        return (s @ v) / s.sum(-1, keepdims=True)

    def transposed(q, k, v, causal=True, eps=0.0):
        T = q.shape[-2]
        S = k @ np.swapaxes(q.conj(), -1, -2)       # roles of Q and K swapped
        s = np.abs(S) ** 2
        s = s * np.tril(np.ones((T, T))) if causal else s
        return (s @ v) / s.sum(-1, keepdims=True)

    def no_square(q, k, v, causal=True, eps=0.0):
        T = q.shape[-2]
        s = np.abs(q @ np.swapaxes(k.conj(), -1, -2))
        s = s * np.tril(np.ones((T, T))) if causal else s
        return (s @ v) / s.sum(-1, keepdims=True)

    def exclusive_mask(q, k, v, causal=True, eps=0.0):
        T = q.shape[-2]
        s = np.abs(q @ np.swapaxes(k.conj(), -1, -2)) ** 2
        s = s * np.tril(np.ones((T, T)), -1) if causal else s
        den = s.sum(-1, keepdims=True)
        return np.where(den == 0, 0, (s @ v) / np.where(den == 0, 1, den))

    return [no_conj, transposed, no_square, exclusive_mask]


@pytest.mark.parametrize("mutant", _mutants(), ids=lambda f: f.__name__)
def test_planted_mistakes_fail_a_pin(mutant):
    """Each plausible slip disagrees with the worked examples or the density-matrix form."""
    failures = 0
    for c in json.load(open(GOLDEN))["cases"]:
        q, k, v = cplx(c["q"]), cplx(c["k"]), cplx(c["v"])
        with np.errstate(all="ignore"):
            got = mutant(q, k, v, causal=True)
        if not np.allclose(got, cplx(c["causal"]["O"]), atol=1e-12):
            failures += 1
    rng = np.random.default_rng(11)
    q, k, v = crandn(rng, 12, 4), crandn(rng, 12, 4), crandn(rng, 12, 4)
    with np.errstate(all="ignore"):
        if not np.allclose(mutant(q, k, v, causal=True), born_attention_density(q, k, v), atol=1e-10):
            failures += 1
    assert failures > 0
