"""Born-rule attention backward, plain fp64 closed form (test infrastructure only).

Gradient convention ("CNet: A Complex-Valued Deep Learning Framework ...",
section 3, the Wirtinger accumulation rule (2) and the CModulus2 worked
example (3)-(5)): a layer receives dL/d(conj O) for a real loss L and returns
dL/d(conj z) for each complex input z.  The map is linear in the incoming
gradient, so the same formulas also give the real-pair gradient
(dL/dRe z + i dL/dIm z = 2 dL/d(conj z)) when the incoming gradient is given
in that form.

Forward (section 11.2, "Closing it: Born-rule attention"):

    S[k, j] = sum_m Q[k, m] conj(K[j, m]),   w[k, j] = |S[k, j]|^2
    l[k]    = sum_{j in J(k)} w[k, j] + eps,  O[k] = sum_{j in J(k)} w[k, j] V[j] / l[k]

With G[k] = dL/d(conj O[k]) and the real per-row scalar delta[k] = Re(G[k]^H O[k]),
differentiating O = N / l and w = S conj(S) gives, for j in J(k):

    D[k, j] = (Re(G[k]^H V[j]) - delta[k]) / l[k]      (dL/dw, up to the 1/2 of the convention)
    dV[j]   = sum_k w[k, j] / l[k] * G[k]
    dQ[k]   = sum_j 2 D[k, j] S[k, j] K[j]
    dK[j]   = sum_k 2 D[k, j] conj(S[k, j]) Q[k]

With the per-head decay (the reading in :mod:`oracle.born`) the weight is
f[k, j] |S[k, j]|^2 with the constant f = gamma^(k - j): every line above takes
f[k, j] as one more factor (in A and in D), since f does not depend on Q or K.

The derivation: dw = 2 Re(conj(S) dS), dS[k, j] = sum_m dQ[k, m] conj(K[j, m]) +
Q[k, m] conj(dK[j, m]); collecting the coefficient of each conj(dz) gives the
lines above.  A row whose denominator l[k] is 0 has O[k] = 0 by definition and
contributes no gradient (the oracle's reading of a 0/0 row).

The pages state that this backward exists in closed form and was checked
against finite differences (section 11.2); they do not print it, so these
formulas are derived here and pinned by finite differences, by torch autograd
of an independent forward, and by the invariances of O.
"""
from __future__ import annotations

import numpy as np

from .born import born_attention, decay_factors


def born_attention_bwd(q, k, v, g, causal: bool = True, eps: float = 0.0, decay=None):
    """(dQ, dK, dV) for complex arrays [..., T, d_h]; g = dL/d(conj O); decay
    as for the forward (causal only)."""
    q = np.asarray(q, dtype=np.complex128)
    k = np.asarray(k, dtype=np.complex128)
    v = np.asarray(v, dtype=np.complex128)
    g = np.asarray(g, dtype=np.complex128)
    T = q.shape[-2]
    o, den = born_attention(q, k, v, causal=causal, eps=eps, return_den=True, decay=decay)
    S = q @ np.swapaxes(k.conj(), -1, -2)                      # S[k, j]
    w = S.real ** 2 + S.imag ** 2
    if decay is not None:
        mask = decay_factors(decay, T)                         # gamma^(k - j) on j <= k
    else:
        mask = np.tril(np.ones((T, T))) if causal else np.ones((T, T))
    live = den != 0.0
    inv = np.where(live, 1.0 / np.where(live, den, 1.0), 0.0)  # 1 / l, 0 for a dead row
    A = w * mask * inv[..., None]                               # w / l on J(k)
    delta = np.sum((g.conj() * o).real, axis=-1)                # Re(G^H O) per row
    E = (g.conj() @ np.swapaxes(v, -1, -2)).real                # Re(G[k]^H V[j])
    D = (E - delta[..., None]) * mask * inv[..., None]
    P = 2.0 * D * S
    dv = np.swapaxes(A, -1, -2).astype(np.complex128) @ g
    dq = P @ k
    dk = np.swapaxes(P.conj(), -1, -2) @ q
    return dq, dk, dv
