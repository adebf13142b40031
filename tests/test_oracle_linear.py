"""Pins for the carried-state Born oracle (CPU only): the step recurrence and
the prefill reproduce the quadratic definition row by row; a sequence split in
two with the first half's state carried equals the whole; the state has the
structure of a sum of outer products (Hermitian, positive semidefinite,
trace = sum |k|^2, M[c] is the v-weighted sum); planted mistakes fail."""
import numpy as np
import pytest

from oracle import born_attention, born_prefill, born_state, born_step


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
