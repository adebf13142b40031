"""Pins for the backward oracle (CPU only).

The backward formulas are derived, not printed on the pages, so each is pinned
by computations that share nothing with it:

* central finite differences of the forward oracle, component by component;
* torch autograd (complex128, CPU) of a forward written here in torch ops;
* the invariances of the forward, which force the gradients to be orthogonal
  to the directions that leave O unchanged;
* planted mistakes (a dropped term, a missing factor, a wrong conjugation),
  each of which must fail the finite-difference pin.

Convention: for L = Re sum conj(G) O the real-pair gradient
dL/dRe z + i dL/dIm z equals the oracle's output for incoming gradient G
(the oracle is linear in G and returns dL/d(conj z) for G = dL/d(conj O)).
"""
import math

import numpy as np
import pytest
import torch

from oracle import born_attention, pct_attention, born_attention_bwd, pct_attention_bwd


def crandn(rng, *shape):
    return (rng.standard_normal(shape) + 1j * rng.standard_normal(shape)) * np.sqrt(0.5)


def fd_grads(fwd, args, g, h=1e-6):
    """Real-pair gradients of L = Re sum conj(g) fwd(*args) by central differences."""
    out = []
    for a_idx, a in enumerate(args):
        grad = np.zeros_like(a)
        it = np.nditer(np.zeros(a.shape), flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            for unit in (1.0, 1j):
                ap, am = a.copy(), a.copy()
                ap[idx] += h * unit
                am[idx] -= h * unit
                lp = np.sum((g.conj() * fwd(*[ap if i == a_idx else x for i, x in enumerate(args)])).real)
                lm = np.sum((g.conj() * fwd(*[am if i == a_idx else x for i, x in enumerate(args)])).real)
                grad[idx] += unit * (lp - lm) / (2 * h)
        out.append(grad)
    return out


BORN_CASES = [(True, 0.0), (False, 0.0), (True, 0.3)]
PCT_CASES = [(True, 0.0), (False, 0.0), (True, -math.log(5.0))]


@pytest.mark.parametrize("causal,eps", BORN_CASES)
def test_born_bwd_matches_finite_differences(causal, eps):
    rng = np.random.default_rng(11)
    T, d = 5, 3
    q, k, v, g = crandn(rng, T, d), crandn(rng, T, d), crandn(rng, T, d), crandn(rng, T, d)
    fd = fd_grads(lambda a, b, c: born_attention(a, b, c, causal=causal, eps=eps), [q, k, v], g)
    got = born_attention_bwd(q, k, v, g, causal=causal, eps=eps)
    for name, x, y in zip("qkv", got, fd):
        np.testing.assert_allclose(x, y, rtol=1e-6, atol=1e-8, err_msg=f"d{name}")


@pytest.mark.parametrize("causal,bias", PCT_CASES)
def test_pct_bwd_matches_finite_differences(causal, bias):
    rng = np.random.default_rng(12)
    T, d = 5, 3
    q, k, v, g = crandn(rng, T, d), crandn(rng, T, d), crandn(rng, T, d), crandn(rng, T, d)
    fd = fd_grads(lambda a, b, c: pct_attention(a, b, c, causal=causal, bias=bias), [q, k, v], g)
    got = pct_attention_bwd(q, k, v, g, causal=causal, bias=bias)
    for name, x, y in zip("qkv", got[:3], fd):
        np.testing.assert_allclose(x, y, rtol=1e-6, atol=1e-8, err_msg=f"d{name}")
    # bias gradient: dL/db by differences of the scalar bias
    h = 1e-6
    lp = np.sum((g.conj() * pct_attention(q, k, v, causal=causal, bias=bias + h)).real)
    lm = np.sum((g.conj() * pct_attention(q, k, v, causal=causal, bias=bias - h)).real)
    np.testing.assert_allclose(got[3].sum(), (lp - lm) / (2 * h), rtol=1e-6, atol=1e-8)


def _torch_born(q, k, v, causal, eps):
    S = q @ k.conj().transpose(-1, -2)
    w = S.real ** 2 + S.imag ** 2
    T = q.shape[-2]
    if causal:
        w = w * torch.tril(torch.ones(T, T, dtype=w.dtype))
    den = w.sum(-1, keepdim=True) + eps
    return (w.to(v.dtype) @ v) / den


def _torch_pct(q, k, v, causal, bias):
    d = q.shape[-1]
    qh = q / torch.sqrt((q.real ** 2 + q.imag ** 2).sum(-1, keepdim=True))
    kh = k / torch.sqrt((k.real ** 2 + k.imag ** 2).sum(-1, keepdim=True))
    s = math.sqrt(d) * (qh @ kh.conj().transpose(-1, -2)).real
    w = torch.sigmoid(s + bias)
    T = q.shape[-2]
    if causal:
        w = w * torch.tril(torch.ones(T, T, dtype=w.dtype))
    return w.to(v.dtype) @ v


@pytest.mark.parametrize("op", ["born", "pct"])
@pytest.mark.parametrize("causal", [True, False])
def test_bwd_matches_torch_autograd(op, causal):
    rng = np.random.default_rng(13)
    B, H, T, d = 2, 2, 33, 8
    q, k, v, g = (crandn(rng, B, H, T, d) for _ in range(4))
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    if op == "born":
        o = _torch_born(tq, tk, tv, causal, 0.0)
        want = born_attention_bwd(q, k, v, g, causal=causal)
    else:
        o = _torch_pct(tq, tk, tv, causal, -0.7)
        want = pct_attention_bwd(q, k, v, g, causal=causal, bias=-0.7)[:3]
    (torch.conj(torch.tensor(g)) * o).real.sum().backward()
    for name, t, w in zip("qkv", (tq, tk, tv), want):
        np.testing.assert_allclose(t.grad.numpy(), w, rtol=1e-10, atol=1e-12, err_msg=f"d{name}")


def _re_dot(a, b):
    return np.sum((a.conj() * b).real, axis=-1)


def _im_dot(a, b):
    return np.sum((a.conj() * b).imag, axis=-1)


def test_born_bwd_invariances():
    """O is unchanged by q_k -> c q_k (any complex c != 0) and by K -> c K, so dQ_k is
    orthogonal to q_k and i q_k, and sum_j <dK_j, k_j> vanishes in both parts;
    rows of the weights sum to one, so sum_j dV_j = sum_k G_k (eps = 0)."""
    rng = np.random.default_rng(14)
    T, d = 40, 6
    q, k, v, g = (crandn(rng, 3, T, d) for _ in range(4))
    for causal in (True, False):
        dq, dk, dv = born_attention_bwd(q, k, v, g, causal=causal)
        scale = np.abs(dq).max()
        assert np.abs(_re_dot(dq, q)).max() < 1e-12 * scale * np.abs(q).max() * d
        assert np.abs(_im_dot(dq, q)).max() < 1e-12 * scale * np.abs(q).max() * d
        sk = np.abs(dk).max() * np.abs(k).max() * d * T
        assert np.abs(_re_dot(dk, k).sum(-1)).max() < 1e-12 * sk
        assert np.abs(_im_dot(dk, k).sum(-1)).max() < 1e-12 * sk
        np.testing.assert_allclose(dv.sum(-2), g.sum(-2), rtol=1e-12, atol=1e-12)


def test_pct_bwd_invariances():
    """O is unchanged by q_i -> lam q_i and k_j -> mu k_j (lam, mu > 0), so dq_i is
    orthogonal to q_i and dk_j to k_j as real 2 d_h-vectors; a zero row gets 0."""
    rng = np.random.default_rng(15)
    T, d = 40, 6
    q, k, v, g = (crandn(rng, T, d) for _ in range(4))
    q[3] = 0.0
    k[7] = 0.0
    for causal in (True, False):
        dq, dk, dv, db = pct_attention_bwd(q, k, v, g, causal=causal, bias=0.4)
        assert np.abs(_re_dot(dq, q)).max() < 1e-12 * np.abs(dq).max() * np.abs(q).max() * d
        assert np.abs(_re_dot(dk, k)).max() < 1e-12 * np.abs(dk).max() * np.abs(k).max() * d
        assert np.all(dq[3] == 0) and np.all(dk[7] == 0)
        # a phase on q_i alone changes O, so the imaginary part is not forced to vanish
        assert np.abs(_im_dot(dq, q)).max() > 1e-3


def test_born_bwd_dead_row_has_no_gradient():
    rng = np.random.default_rng(16)
    T, d = 6, 3
    q, k, v, g = (crandn(rng, T, d) for _ in range(4))
    q[2] = 0.0                                   # S[2, :] = 0 -> l[2] = 0 -> O[2] = 0
    dq, dk, dv = born_attention_bwd(q, k, v, g, causal=True)
    assert np.all(dq[2] == 0)
    g2 = g.copy()
    g2[2] = 123.0 + 45j                          # the dead row's incoming gradient is ignored
    for a, b in zip((dq, dk, dv), born_attention_bwd(q, k, v, g2, causal=True)):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


def _born_mutants():
    def base(q, k, v, g, causal, eps, delta=True, two=2.0, conj_k=True):
        o, den = born_attention(q, k, v, causal=causal, eps=eps, return_den=True)
        T = q.shape[-2]
        S = q @ k.conj().T
        w = np.abs(S) ** 2
        mask = np.tril(np.ones((T, T))) if causal else np.ones((T, T))
        A = w * mask / den[:, None]
        dl = np.sum((g.conj() * o).real, -1) if delta else 0.0
        D = ((g.conj() @ v.T).real - (dl[:, None] if delta else 0.0)) * mask / den[:, None]
        P = two * D * S
        return P @ k, (P.conj().T if conj_k else P.T) @ q, A.T @ g

    return {
        "none": base,
        "no_delta": lambda *a: base(*a, delta=False),
        "no_factor_two": lambda *a: base(*a, two=1.0),
        "dk_unconjugated": lambda *a: base(*a, conj_k=False),
    }


def _pct_mutants():
    def base(q, k, v, g, causal, bias, project=True, dsig=True):
        T, d = q.shape
        nq = np.linalg.norm(q, axis=-1, keepdims=True)
        nk = np.linalg.norm(k, axis=-1, keepdims=True)
        qh, kh = q / nq, k / nk
        s = math.sqrt(d) * (qh @ kh.conj().T).real
        w = 1 / (1 + np.exp(-(s + bias)))
        mask = np.tril(np.ones((T, T))) if causal else np.ones((T, T))
        w = w * mask
        ds = (g.conj() @ v.T).real * (w * (1 - w) if dsig else w) * mask
        gq = math.sqrt(d) * ds @ kh
        gk = math.sqrt(d) * ds.T @ qh
        if project:
            gq = gq - np.sum((gq.conj() * qh).real, -1, keepdims=True) * qh
            gk = gk - np.sum((gk.conj() * kh).real, -1, keepdims=True) * kh
        return gq / nq, gk / nk, w.T @ g

    return {
        "none": base,
        "no_projection": lambda *a: base(*a, project=False),
        "sigmoid_not_derivative": lambda *a: base(*a, dsig=False),
    }


@pytest.mark.parametrize("name", list(_born_mutants()))
def test_born_planted_mistakes_fail_fd(name):
    rng = np.random.default_rng(17)
    T, d = 5, 3
    q, k, v, g = (crandn(rng, T, d) for _ in range(4))
    fd = fd_grads(lambda a, b, c: born_attention(a, b, c, causal=True), [q, k, v], g)
    got = _born_mutants()[name](q, k, v, g, True, 0.0)
    fails = any(not np.allclose(x, y, rtol=1e-6, atol=1e-8) for x, y in zip(got, fd))
    assert fails == (name != "none")   # the unmutated formula, written the same way, passes


@pytest.mark.parametrize("name", list(_pct_mutants()))
def test_pct_planted_mistakes_fail_fd(name):
    rng = np.random.default_rng(18)
    T, d = 5, 3
    q, k, v, g = (crandn(rng, T, d) for _ in range(4))
    fd = fd_grads(lambda a, b, c: pct_attention(a, b, c, causal=True), [q, k, v], g)
    got = _pct_mutants()[name](q, k, v, g, True, 0.0)
    fails = any(not np.allclose(x, y, rtol=1e-6, atol=1e-8) for x, y in zip(got, fd))
    assert fails == (name != "none")
