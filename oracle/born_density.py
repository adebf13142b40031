"""Born attention through density-matrix prefix states (test infrastructure only).

A second formulation, used only to pin :mod:`oracle.born`.  The Born score is
a linear functional of the key's density matrix: for rho_j = k_j k_j^H
(rank one, Hermitian, positive semidefinite -- "The Quantum Shortcut",
section 2, "Complex states and the density matrix" and "The Born rule"),

    |<q, k_j>|^2 = q^H rho_j q .

Summing over the causal prefix gives the exact finite feature map that the
CNet BornAttention layer uses for its linear mode ("Show HN: CNET",
BornAttention: each key lifted to its outer product, a carried state):

    Z_t      = sum_{j <= t} rho_j                (normaliser state)
    M_t[c]   = sum_{j <= t} V[j, c] rho_j        (one state per value channel)
    O[t, c]  = (q_t^H M_t[c] q_t) / (q_t^H Z_t q_t + eps)

The states are carried token by token (O(T d_h^3) per head), with no T x T
matrix anywhere, so this shares no step with the quadratic definition.
"""
from __future__ import annotations

import numpy as np


def born_attention_density(q, k, v, causal: bool = True, eps: float = 0.0):
    """q, k, v: complex arrays [T, d_h] (one head).  Returns complex128 [T, d_h]."""
    q = np.asarray(q, dtype=np.complex128)
    k = np.asarray(k, dtype=np.complex128)
    v = np.asarray(v, dtype=np.complex128)
    T, d = q.shape
    Z = np.zeros((d, d), dtype=np.complex128)
    M = np.zeros((d, d, d), dtype=np.complex128)   # M[c] is a d x d state
    out = np.zeros((T, d), dtype=np.complex128)

    def read(t):
        qt = q[t]
        den = (qt.conj() @ Z @ qt).real + eps
        if den == 0.0:
            return np.zeros(d, dtype=np.complex128)
        num = np.array([qt.conj() @ M[c] @ qt for c in range(d)])
        return num / den

    if causal:
        for t in range(T):
            rho = np.outer(k[t], k[t].conj())
            Z += rho
            M += v[t][:, None, None] * rho[None, :, :]
            out[t] = read(t)
    else:
        for t in range(T):
            rho = np.outer(k[t], k[t].conj())
            Z += rho
            M += v[t][:, None, None] * rho[None, :, :]
        for t in range(T):
            out[t] = read(t)
    return out
