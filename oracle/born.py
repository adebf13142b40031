"""Born-rule attention, plain fp64 definition (test infrastructure only).

Definition ("CNet: A Complex-Valued Deep Learning Framework with Wirtinger
Autodifferentiation and FFT-Hadamard Convolution", section 11.2, paragraph
"Closing it: Born-rule attention", and Figure 2; the same operator with a
per-query temperature that cancels in the ratio is eq. (5) of "The Quantum
Shortcut", section 5.5):

    S[k, j] = <Q_k, K_j> = sum_m Q[k, m] * conj(K[j, m])
    s[k, j] = |S[k, j]|^2                       (Born-rule measurement)
    A[k, j] = s[k, j] / sum_{j' in J(k)} s[k, j']
    O[k]    = sum_{j in J(k)} A[k, j] V[j]

with J(k) = {0..k} when causal, else all keys.  The Hermitian inner product
conjugates the key side ("The Quantum Shortcut", section 2: the bra is the
conjugate transpose); for |S|^2 the choice of side does not matter, the
conjugation itself does.

Readings where the pages are silent (each also listed in the design notes):
* ``eps`` (the BornAttention layer's argument, "Show HN: CNET") is added to
  the row denominator: A = s / (sum s + eps); default 0.
* A row whose denominator is exactly 0 returns O = 0.
* ``decay`` ("Show HN: CNET", BornAttention: a fixed per-head decay that
  multiplies the score, the formula itself lost in the page's text; the same
  page runs it together with the linear form on PG-19, so it must survive the
  carried-state recursion): causal only, with a per-head gamma in (0, 1] the
  weight of key j for query k is

      w[k, j] = gamma ** (k - j) * |S[k, j]|^2,   j <= k,

  which is the one fixed per-head factor of the score that the recursion
  Z <- gamma Z + k k^H reproduces.  gamma = 1 is plain Born attention.
"""
from __future__ import annotations

import numpy as np


def _as_c128(x):
    return np.asarray(x, dtype=np.complex128)


def decay_factors(decay, T: int):
    """gamma ** (k - j) on j <= k, 0 above the diagonal: [..., T, T] for a
    gamma of shape [...] (a scalar, or one value per head)."""
    g = np.asarray(decay, dtype=np.float64)
    if np.any(~(g > 0.0)) or np.any(g > 1.0):
        raise ValueError("decay must lie in (0, 1]")
    dist = np.arange(T)[:, None] - np.arange(T)[None, :]          # k - j
    return np.where(dist >= 0, g[..., None, None] ** np.maximum(dist, 0), 0.0)


def born_attention(q, k, v, causal: bool = True, eps: float = 0.0, return_den: bool = False, decay=None):
    """O for every query row.  q, k, v: complex arrays [..., T, d_h].  decay:
    None, or gamma broadcastable to the leading dimensions [...] (e.g. [H]
    for [B, H, T, d_h]); causal only."""
    q, k, v = _as_c128(q), _as_c128(k), _as_c128(v)
    T = q.shape[-2]
    S = q @ np.swapaxes(k.conj(), -1, -2)            # [..., T, T]: S[k, j] = <q_k, k_j>
    s = S.real ** 2 + S.imag ** 2                     # |S|^2
    if decay is not None:
        if not causal:
            raise ValueError("decay is defined for causal attention only")
        s = s * decay_factors(decay, T)               # gamma^(k - j), 0 for j > k
    elif causal:
        s = s * np.tril(np.ones((T, T)))              # keep j <= k
    den = s.sum(axis=-1) + eps                        # [..., T]
    num = s.astype(np.complex128) @ v                 # sum_j s[k, j] V[j]
    safe = np.where(den == 0.0, 1.0, den)
    out = np.where((den == 0.0)[..., None], 0.0, num / safe[..., None])
    return (out, den) if return_den else out


def born_attention_rows(q, k, v, rows, causal: bool = True, eps: float = 0.0, decay=None):
    """O for selected rows only.

    q, k, v: complex arrays [B, H, T, d_h]; rows: integer array [n, 3] of
    (b, h, t); decay: None or gamma per head [H] (causal only).  Returns
    complex128 [n, d_h].  Each row is computed on its own from the same
    definition, so full-size outputs can be sampled cheaply.
    """
    if decay is not None:
        if not causal:
            raise ValueError("decay is defined for causal attention only")
        gam = np.broadcast_to(np.asarray(decay, dtype=np.float64), (q.shape[1],))
        if np.any(~(gam > 0.0)) or np.any(gam > 1.0):
            raise ValueError("decay must lie in (0, 1]")
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    out = np.zeros((rows.shape[0], q.shape[-1]), dtype=np.complex128)
    for i, (b, h, t) in enumerate(rows):
        qr = _as_c128(q[b, h, t])
        J = t + 1 if causal else k.shape[2]
        kk = _as_c128(k[b, h, :J])
        vv = _as_c128(v[b, h, :J])
        S = kk.conj() @ qr                            # S[j] = sum_m q[m] conj(k[j, m])
        s = S.real ** 2 + S.imag ** 2
        if decay is not None:
            s = s * gam[h] ** (t - np.arange(J))       # gamma^(t - j)
        den = s.sum() + eps
        out[i] = 0.0 if den == 0.0 else (s @ vv) / den
    return out
