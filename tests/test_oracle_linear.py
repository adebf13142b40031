"""Pins for the carried-state Born oracle (CPU only): the step recurrence and
the prefill reproduce the quadratic definition row by row; a sequence split in
two with the first half's state carried equals the whole; the state has the
structure of a sum of outer products (Hermitian, positive semidefinite,
trace = sum |k|^2, M[c] is the v-weighted sum); planted mistakes fail."""
import numpy as np
import pytest

from oracle import (born_attention, born_prefill, born_state, born_step, pack_hermitian, pack_state,
                    unpack_hermitian, unpack_state)


def crandn(rng, *shape):
    return (rng.standard_normal(shape) + 1j * rng.standard_normal(shape)) * np.sqrt(0.5)


@pytest.mark.parametrize("eps", [0.0, 0.3])
def test_prefill_from_zero_is_the_quadratic_definition(eps):
    rng = np.random.default_rng(71)
    T, d = 30, 5
    q, k, v = crandn(rng, T, d), crandn(rng, T, d), crandn(rng, T, d)
    out, Z, M = born_prefill(q, k, v, eps=eps)
    np.testing.assert_allclose(out, born_attention(q, k, v, causal=True, eps=eps), rtol=1e-11, atol=1e-13)


def test_carry_splits_a_sequence():
    rng = np.random.default_rng(72)
    T, d, cut = 40, 4, 17
    q, k, v = crandn(rng, T, d), crandn(rng, T, d), crandn(rng, T, d)
    Z1, M1 = born_state(k[:cut], v[:cut])
    out2, Z2, M2 = born_prefill(q[cut:], k[cut:], v[cut:], Z1, M1)
    full = born_attention(q, k, v, causal=True)
    np.testing.assert_allclose(out2, full[cut:], rtol=1e-11, atol=1e-13)
    Zf, Mf = born_state(k, v)
    np.testing.assert_allclose(Z2, Zf, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(M2, Mf, rtol=1e-12, atol=1e-12)


def test_state_structure():
    rng = np.random.default_rng(73)
    T, d = 25, 6
    k, v = crandn(rng, T, d), crandn(rng, T, d)
    Z, M = born_state(k, v)
    np.testing.assert_allclose(Z, Z.conj().T, rtol=0, atol=1e-12)
    assert np.linalg.eigvalsh(Z).min() > -1e-10
    np.testing.assert_allclose(np.trace(Z).real, np.sum(np.abs(k) ** 2), rtol=1e-12)
    # M[c] is the V[:, c]-weighted sum of the same outer products; its trace is sum_j V[j, c] |k_j|^2
    np.testing.assert_allclose(np.trace(M, axis1=1, axis2=2), (np.abs(k) ** 2).sum(-1) @ v, rtol=1e-12)
    # with every V row equal to c, M[c'] = c_{c'} Z
    c = crandn(rng, d)
    _, Mc = born_state(k, np.broadcast_to(c, (T, d)))
    np.testing.assert_allclose(Mc, c[:, None, None] * Z[None], rtol=1e-12, atol=1e-12)


def test_step_hand_example():
    # d = 1: Z = sum |k|^2, M = sum v |k|^2, o = M / Z (q cancels)
    Z, M = born_state(np.array([[2.0 + 0j]]), np.array([[3.0 + 1j]]))
    o, Z, M = born_step(np.array([0.5j]), np.array([1.0 + 0j]), np.array([-1.0 + 0j]), Z, M)
    np.testing.assert_allclose(o, [((3 + 1j) * 4 - 1) / 5], rtol=1e-14)


def test_planted_mistakes_fail():
    rng = np.random.default_rng(74)
    T, d = 12, 3
    q, k, v = crandn(rng, T, d), crandn(rng, T, d), crandn(rng, T, d)
    want = born_attention(q, k, v, causal=True)
    # reading out before adding the current token (an exclusive prefix)
    Z = np.zeros((d, d), complex)
    M = np.zeros((d, d, d), complex)
    bad = []
    for t in range(T):
        den = (q[t].conj() @ Z @ q[t]).real
        bad.append(np.zeros(d) if den == 0 else np.einsum("a,cab,b->c", q[t].conj(), M, q[t]) / den)
        Z, M = born_state(k[t:t + 1], v[t:t + 1], Z, M)
    assert not np.allclose(np.array(bad), want)
    # the outer product unconjugated (k k^T)
    Z2 = sum(np.outer(k[j], k[j]) for j in range(T))
    assert not np.allclose(q[-1].conj() @ Z2 @ q[-1], q[-1].conj() @ born_state(k, v)[0] @ q[-1])


def test_packed_hermitian_hand_example():
    # k = (1, i): k k^H = [[1, -i], [i, 1]]; Re above and on the diagonal, Im of the upper entry below
    X = np.outer([1, 1j], np.conj([1, 1j]))
    np.testing.assert_array_equal(X, [[1, -1j], [1j, 1]])
    np.testing.assert_array_equal(pack_hermitian(X), [[1.0, 0.0], [-1.0, 1.0]])
    np.testing.assert_array_equal(unpack_hermitian([[1.0, 0.0], [-1.0, 1.0]]), X)


def test_packed_state_round_trip_and_parts():
    rng = np.random.default_rng(75)
    T, d = 20, 5
    k, v = crandn(rng, T, d), crandn(rng, T, d)
    Z, M = born_state(k, v)
    S = pack_state(Z, M)
    assert S.shape == (2 * d + 1, d, d) and S.dtype == np.float64
    Z2, M2 = unpack_state(S)
    np.testing.assert_allclose(Z2, Z, rtol=0, atol=1e-12)
    np.testing.assert_allclose(M2, M, rtol=0, atol=1e-12)
    # the parts are the real- and imaginary-V-weighted sums of outer products
    ZR, MR = born_state(k, v.real.astype(complex))
    ZI, MI = born_state(k, v.imag.astype(complex))
    for c in range(d):
        np.testing.assert_allclose(S[c], pack_hermitian(MR[c]), rtol=0, atol=1e-12)
        np.testing.assert_allclose(S[d + c], pack_hermitian(MI[c]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(S[2 * d], pack_hermitian(Z), rtol=0, atol=1e-12)


def test_packed_form_carries_the_quadratic_form():
    """q^H X q = sum_a |q_a|^2 P[a, a] + 2 sum_{a != b} phi_ab(q) P[a, b] with
    phi_ab(q) = Re(q_a conj q_b) for a < b and Im(q_b conj q_a) for a > b: the
    identity a packed-state readout relies on."""
    rng = np.random.default_rng(76)
    d = 7
    k = crandn(rng, 9, d)
    X = sum(np.outer(kj, kj.conj()) * w for kj, w in zip(k, rng.standard_normal(9)))
    P = pack_hermitian(X)
    for _ in range(5):
        q = crandn(rng, d)
        phi = np.empty((d, d))
        for a in range(d):
            for b in range(d):
                phi[a, b] = (q[a] * np.conj(q[b])).real if a <= b else (q[b] * np.conj(q[a])).imag
        weight = np.where(np.eye(d, dtype=bool), 1.0, 2.0)
        np.testing.assert_allclose((weight * phi * P).sum(), (q.conj() @ X @ q).real, rtol=1e-12)
        # and the packed outer product is phi itself: P(q q^H) = phi(q)
        np.testing.assert_allclose(pack_hermitian(np.outer(q, q.conj())), phi, rtol=0, atol=1e-14)


def test_planted_packing_mistake_fails():
    # storing the lower triangle as +Im of the lower entry (the transpose's sign) breaks the round trip
    rng = np.random.default_rng(77)
    q = crandn(rng, 4)
    X = np.outer(q, q.conj())
    wrong = np.where(np.triu(np.ones((4, 4), bool)), X.real, X.imag)
    assert np.abs(unpack_hermitian(wrong) - X).max() > 1e-3
