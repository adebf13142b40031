"""Rotary phase embedding, plain fp64 definition (test infrastructure only).

"Show HN: CNET", the RotaryEmbed layer: position enters as a complex phase
rotation of each component, with base 10000, and an absolute position (setPos)
for the one-token step mode.  Written out:

    y[t, m] = x[t, m] * exp(i (p0 + t) theta_m),   theta_m = base ** (-m / d_h)

for token t = 0..T-1 of a [..., T, d_h] tensor and channel m = 0..d_h-1.
The rotation is the plainest reading of "phase rotation by position" with the
usual RoPE frequencies; the page gives the base but not the exponent's form,
so theta_m = base^(-m/d_h) over the d_h complex channels is a reading (each
complex channel is one rotation plane).
"""
from __future__ import annotations

import numpy as np


def rotary(x, pos0: int = 0, base: float = 10000.0):
    x = np.asarray(x, dtype=np.complex128)
    T, d = x.shape[-2], x.shape[-1]
    theta = base ** (-np.arange(d, dtype=np.float64) / d)
    pos = pos0 + np.arange(T, dtype=np.float64)
    return x * np.exp(1j * pos[:, None] * theta[None, :])
