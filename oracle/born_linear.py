"""Born attention with a carried density state: state build, prefill with an
incoming state, and the one-token step (test infrastructure only).

"Show HN: CNET", BornAttention (linear and step modes): each key is lifted
to its outer product and a running state is carried along the sequence, so
memory grows linearly, the result is exact (the feature map is finite), and
decoding processes a single token per call while updating that state in
place, at constant memory.  "The Quantum Shortcut", section 2: the Born rule
as the linear functional q^H rho q of the density matrix rho = k k^H.  Per
head:

    Z      = sum_j k_j k_j^H                   (d x d, the normaliser state)
    M[c]   = sum_j V[j, c] k_j k_j^H            (d x d for each value channel c)
    O[t, c] = q_t^H M_t[c] q_t / (q_t^H Z_t q_t + eps)

where the states at token t hold every key j <= t (the carried state plus the
tokens of the current call up to t).  Arrays here are per head: q, k, v
[T, d]; Z [d, d]; M [d, d, d] indexed M[c, a, b].

Decay (the reading of BornAttention's fixed per-head decay, see
:mod:`oracle.born`): with gamma in (0, 1] each token first scales the state
by gamma and then adds its own outer product,

    Z_t = gamma Z_{t-1} + k_t k_t^H,   M_t[c] = gamma M_{t-1}[c] + V[t, c] k_t k_t^H,

so Z_t = sum_{j <= t} gamma^(t - j) k_j k_j^H and the read-out q_t^H M_t q_t /
q_t^H Z_t q_t is the decayed quadratic form.  gamma = 1 is the plain state.

Packed real form of the state (the layout the device library carries).  Z is
Hermitian and each M[c] splits into two Hermitian parts,
M[c] = X_c + i X_{d+c} with X_c = (M[c] + M[c]^H) / 2 and
X_{d+c} = (M[c] - M[c]^H) / (2i) (the sums of k k^H weighted by Re V[:, c] and
by Im V[:, c]); X_{2d} = Z.  A Hermitian d x d matrix X has d^2 real degrees
of freedom, stored as a real d x d matrix P with P[a, b] = Re X[a, b] for
a <= b and P[a, b] = Im X[b, a] for a > b.  The packed state is S[n] = P(X_n)
for n = 0 .. 2d, shape [2d + 1, d, d].
"""
from __future__ import annotations

import numpy as np


def _c(x):
    return np.asarray(x, dtype=np.complex128)


def _gamma(gamma):
    g = float(gamma)
    if not (0.0 < g <= 1.0):
        raise ValueError("decay must lie in (0, 1]")
    return g


def born_state(k, v, Z0=None, M0=None, gamma: float = 1.0):
    """(Z, M) after adding every token of k, v [T, d] to the state (Z0, M0)
    (zero if None), one token at a time: scale by gamma, add k k^H."""
    g = _gamma(gamma)
    k, v = _c(k), _c(v)
    d = k.shape[-1]
    Z = np.zeros((d, d), np.complex128) if Z0 is None else _c(Z0).copy()
    M = np.zeros((d, d, d), np.complex128) if M0 is None else _c(M0).copy()
    for j in range(k.shape[0]):
        rho = np.outer(k[j], k[j].conj())
        Z = g * Z + rho
        M = g * M + v[j][:, None, None] * rho[None, :, :]
    return Z, M


def born_step(q, k, v, Z, M, eps: float = 0.0, gamma: float = 1.0):
    """One token: add (k, v) to the state (after scaling it by gamma), then
    read out q.  q, k, v [d].  Returns (o [d], Z', M'); o = 0 when the
    denominator is 0."""
    q = _c(q)
    Z, M = born_state(_c(k)[None, :], _c(v)[None, :], Z, M, gamma)
    den = (q.conj() @ Z @ q).real + eps
    if den == 0.0:
        return np.zeros(q.shape[-1], np.complex128), Z, M
    num = np.einsum("a,cab,b->c", q.conj(), M, q)
    return num / den, Z, M


def born_prefill(q, k, v, Z0=None, M0=None, eps: float = 0.0, gamma: float = 1.0):
    """Causal Born over a sequence whose keys before token 0 are summarised by
    the state (Z0, M0): each token is one step.  Returns (O [T, d], Z, M)."""
    q, k, v = _c(q), _c(k), _c(v)
    d = q.shape[-1]
    Z = np.zeros((d, d), np.complex128) if Z0 is None else _c(Z0)
    M = np.zeros((d, d, d), np.complex128) if M0 is None else _c(M0)
    out = np.zeros(q.shape, np.complex128)
    for t in range(q.shape[0]):
        out[t], Z, M = born_step(q[t], k[t], v[t], Z, M, eps, gamma)
    return out, Z, M


def pack_hermitian(X):
    """P(X) for a Hermitian X [d, d]: Re on and above the diagonal, Im of the
    transposed entry below it."""
    X = _c(X)
    up = np.triu(np.ones(X.shape, bool))
    return np.where(up, X.real, X.T.imag)


def unpack_hermitian(P):
    """The Hermitian X whose packed form is P."""
    P = np.asarray(P, dtype=np.float64)
    d = P.shape[-1]
    X = np.zeros((d, d), np.complex128)
    for a in range(d):
        X[a, a] = P[a, a]
        for b in range(a + 1, d):
            X[a, b] = P[a, b] + 1j * P[b, a]
            X[b, a] = np.conj(X[a, b])
    return X


def pack_state(Z, M):
    """Packed real state S [2d + 1, d, d] of (Z, M)."""
    Z, M = _c(Z), _c(M)
    d = Z.shape[-1]
    S = np.zeros((2 * d + 1, d, d))
    for c in range(d):
        S[c] = pack_hermitian((M[c] + M[c].conj().T) / 2)
        S[d + c] = pack_hermitian((M[c] - M[c].conj().T) / 2j)
    S[2 * d] = pack_hermitian(Z)
    return S


def unpack_state(S):
    """(Z, M) of a packed state S [2d + 1, d, d]."""
    S = np.asarray(S, dtype=np.float64)
    d = S.shape[-1]
    M = np.stack([unpack_hermitian(S[c]) + 1j * unpack_hermitian(S[d + c]) for c in range(d)])
    return unpack_hermitian(S[2 * d]), M
