"""Phase-coherent (PCT) attention, plain fp64 definition (test infrastructure only).

Definition ("Complex-valued Phase-Coherent Transformers", section 1, the
scaled cosine score, and Appendix D.2, the PCT cell): queries and keys are
each divided by their complex L2 norm, the score is the real part of their
Hermitian inner product scaled by sqrt(d_h), the gate is an element-wise
sigmoid with an additive bias, and the real weights multiply complex values
with no row normalisation (keys do not compete, section 2.2):

    qh_i = q_i / ||q_i||,   kh_j = k_j / ||k_j||
    s[i, j] = sqrt(d_h) * Re sum_m qh[i, m] * conj(kh[j, m])
    w[i, j] = 1 / (1 + exp(-(s[i, j] + b)))
    O[i]    = sum_{j in J(i)} w[i, j] V[j]

J(i) = {0..i} when causal, else all keys.  The bar over q and k in the
pages' score denotes the normalised vector, not a conjugate (the text says
the vectors are divided by their modulus).

Readings where the pages are silent:
* a zero-norm q or k has inverse norm 0, so its scores are 0 and w = sigmoid(b);
* the bias b is a plain argument (the pages initialise it to -log N; the
  default here is 0, a plain sigmoid of the score).
"""
from __future__ import annotations

import math
import numpy as np


def _unit(x):
    x = np.asarray(x, dtype=np.complex128)
    n = np.sqrt(np.sum(x.real ** 2 + x.imag ** 2, axis=-1, keepdims=True))
    inv = np.where(n == 0.0, 0.0, 1.0 / np.where(n == 0.0, 1.0, n))
    return x * inv


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def pct_scores(q, k):
    """s = sqrt(d_h) Re <q_i/||q_i||, k_j/||k_j||>, shape [..., T, T]."""
    d = q.shape[-1]
    S = _unit(q) @ np.swapaxes(_unit(k).conj(), -1, -2)
    return math.sqrt(d) * S.real


def pct_attention(q, k, v, causal: bool = False, bias: float = 0.0):
    """O for every query row.  q, k, v: complex arrays [..., T, d_h]."""
    v = np.asarray(v, dtype=np.complex128)
    T = q.shape[-2]
    w = _sigmoid(pct_scores(q, k) + bias)
    if causal:
        w = w * np.tril(np.ones((T, T)))
    return w.astype(np.complex128) @ v


def pct_attention_rows(q, k, v, rows, causal: bool = False, bias: float = 0.0):
    """O for selected (b, h, t) rows of [B, H, T, d_h] inputs; complex128 [n, d_h]."""
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    d = q.shape[-1]
    out = np.zeros((rows.shape[0], d), dtype=np.complex128)
    for i, (b, h, t) in enumerate(rows):
        J = t + 1 if causal else k.shape[2]
        qh = _unit(q[b, h, t])
        kh = _unit(k[b, h, :J])
        s = math.sqrt(d) * (kh.conj() @ qh).real
        w = _sigmoid(s + bias)
        out[i] = w @ np.asarray(v[b, h, :J], dtype=np.complex128)
    return out


# ---------------------------------------------------------------------------- siblings
# "Complex-valued Phase-Coherent Transformers", Appendix D.2: two further
# members of the family use the same scaled cosine score.  The L2-softmax cell
# normalises exp(s) over the keys of a row where the PCT cell applies an
# independent sigmoid per key; the complex screening cell gates each score by
# r^2 relu(s - t)^2.  Only the weight map differs.  The
# screening cell's TanhNorm of the aggregate and its modReLU Hadamard gate act
# after the attention sum and are not part of it.


def pct_softmax_attention(q, k, v, causal: bool = False):
    """L2-softmax member: w[i, j] = exp(s[i, j]) / sum_{j' in J(i)} exp(s[i, j']).

    The score is bounded by sqrt(d_h) (Cauchy-Schwarz), so exp(s) needs no
    shift to stay finite; the definition is written as it reads.
    """
    v = np.asarray(v, dtype=np.complex128)
    T = q.shape[-2]
    e = np.exp(pct_scores(q, k))
    if causal:
        e = e * np.tril(np.ones((T, T)))
    w = e / e.sum(axis=-1, keepdims=True)
    return w.astype(np.complex128) @ v


def pct_screen_attention(q, k, v, causal: bool = False, r: float = 1.0, t: float = 0.0):
    """Screening gate core: w[i, j] = r^2 max(s[i, j] - t, 0)^2, no row normalisation."""
    v = np.asarray(v, dtype=np.complex128)
    T = q.shape[-2]
    w = r * r * np.maximum(pct_scores(q, k) - t, 0.0) ** 2
    if causal:
        w = w * np.tril(np.ones((T, T)))
    return w.astype(np.complex128) @ v
