"""Phase-coherent (PCT) attention backward, plain fp64 closed form (test infrastructure only).

Gradient convention as in :mod:`oracle.born_grad` ("CNet ...", section 3,
rule (2)): given G[i] = dL/d(conj O[i]), return dL/d(conj z) for q, k, v; the
formulas are linear in G, so they also hold for real-pair gradients.

Forward ("Complex-valued Phase-Coherent Transformers", section 1 and
Appendix D.2): qh = q / ||q||, kh = k / ||k||,
s[i, j] = sqrt(d_h) Re sum_m qh[i, m] conj(kh[j, m]),  w = sigmoid(s + b),
O[i] = sum_{j in J(i)} w[i, j] V[j].

Backward, for j in J(i):

    dV[j]     = sum_i w[i, j] G[i]
    ds[i, j]  = Re(G[i]^H V[j]) * w[i, j] (1 - w[i, j])
    gqh[i]    = sqrt(d_h) sum_j ds[i, j] kh[j]        (the score is the real inner
    gkh[j]    = sqrt(d_h) sum_i ds[i, j] qh[i]         product of qh and kh as 2 d_h-vectors)
    dq[i]     = (gqh[i] - Re(gqh[i]^H qh[i]) qh[i]) / ||q[i]||
    dk[j]     = (gkh[j] - Re(gkh[j]^H kh[j]) kh[j]) / ||k[j]||
    db_row[i] = sum_{j in J(i)} ds[i, j]               (bias gradient, per query row)

The last two lines are the derivative of x -> x / ||x|| on R^{2 d_h}: the
component along x is removed and the rest divided by ||x||.  A zero-norm q or
k (whose normalised vector is 0 by the forward's reading) gets gradient 0.
The pages do not print a backward; these lines are derived here and pinned by
finite differences, torch autograd and the scale invariance of O.
"""
from __future__ import annotations

import math
import numpy as np


def _norm_and_unit(x):
    x = np.asarray(x, dtype=np.complex128)
    n = np.sqrt(np.sum(x.real ** 2 + x.imag ** 2, axis=-1, keepdims=True))
    inv = np.where(n == 0.0, 0.0, 1.0 / np.where(n == 0.0, 1.0, n))
    return x * inv, inv


def pct_attention_bwd(q, k, v, g, causal: bool = False, bias: float = 0.0):
    """(dQ, dK, dV, db_rows) for complex arrays [..., T, d_h]; g = dL/d(conj O)."""
    v = np.asarray(v, dtype=np.complex128)
    g = np.asarray(g, dtype=np.complex128)
    T, d = q.shape[-2], q.shape[-1]
    qh, rq = _norm_and_unit(q)
    kh, rk = _norm_and_unit(k)
    s = math.sqrt(d) * (qh @ np.swapaxes(kh.conj(), -1, -2)).real
    w = 1.0 / (1.0 + np.exp(-(s + bias)))
    mask = np.tril(np.ones((T, T))) if causal else np.ones((T, T))
    w = w * mask
    E = (g.conj() @ np.swapaxes(v, -1, -2)).real                # Re(G[i]^H V[j])
    ds = E * w * (1.0 - w) * mask
    dv = np.swapaxes(w, -1, -2).astype(np.complex128) @ g
    gqh = math.sqrt(d) * (ds.astype(np.complex128) @ kh)
    gkh = math.sqrt(d) * (np.swapaxes(ds, -1, -2).astype(np.complex128) @ qh)
    dq = (gqh - np.sum((gqh.conj() * qh).real, axis=-1, keepdims=True) * qh) * rq
    dk = (gkh - np.sum((gkh.conj() * kh).real, axis=-1, keepdims=True) * kh) * rk
    db_rows = ds.sum(axis=-1)
    return dq, dk, dv, db_rows
