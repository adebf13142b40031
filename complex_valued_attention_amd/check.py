"""Host/device transfer helpers and the parity error measure.

Nothing here computes attention.  ``rowwise_rel_err`` is the error measure
used against the oracle: for every output row (one query of one head) the
largest complex deviation divided by the row's largest reference modulus,
maximised over rows.  Element-wise relative error is ill-posed for these
operators (outputs are combinations of random values and have entries near
zero), the row-wise form keeps the scale of each query's output.
"""
from __future__ import annotations

import numpy as np

from .inputs import Inputs, bf16_bits_to_f64

# Parity bars: fp32 arithmetic on complex64 inputs, bf16 products with fp32 accumulation.
TOL = {"c64": 1e-4, "bf16": 2e-2}
# Row-scale floor for gradient comparisons (fraction of the tensor's largest row scale).
GRAD_FLOOR = 1e-3


def rowwise_rel_err(got: np.ndarray, ref: np.ndarray, floor: float = 0.0) -> float:
    """Max over rows of max |got - ref| / max |ref| in the row.

    ``floor`` > 0 raises each row's scale to at least ``floor`` times the
    largest row scale of the tensor.  Gradients use it: some of their rows are
    exactly zero in exact arithmetic (Born's first causal row of dQ), and those
    are measured by their absolute error at the tensor's scale.
    """
    got = np.asarray(got, dtype=np.complex128).reshape(-1, ref.shape[-1])
    ref = np.asarray(ref, dtype=np.complex128).reshape(-1, ref.shape[-1])
    diff = np.abs(got - ref).max(axis=1)
    scale = np.abs(ref).max(axis=1)
    if floor > 0.0 and scale.size:
        scale = np.maximum(scale, floor * scale.max())
    if np.any(~np.isfinite(diff)):
        return float("inf")
    zero = scale == 0.0
    err = np.where(zero, np.where(diff == 0.0, 0.0, np.inf), diff / np.where(zero, 1.0, scale))
    return float(err.max()) if err.size else 0.0


def to_device(inp: Inputs, device="cuda"):
    """Upload the rounded inputs: complex64 tensors, or (re, im) bf16 plane pairs."""
    import torch
    if inp.layout == "c64":
        return tuple(torch.from_numpy(inp.dev[n]).to(device) for n in ("q", "k", "v"))
    out = []
    for n in ("q", "k", "v"):
        pair = tuple(torch.from_numpy(inp.dev[f"{n}_{p}"].view(np.int16)).to(device).view(torch.bfloat16)
                     for p in ("re", "im"))
        out.append(pair)
    return tuple(out)


def grad_to_device(g, device="cuda"):
    """Upload an incoming gradient (``inputs.Grad``) in its layout."""
    import torch
    if g.layout == "c64":
        return torch.from_numpy(g.dev["g"]).to(device)
    return tuple(torch.from_numpy(g.dev[f"g_{p}"].view(np.int16)).to(device).view(torch.bfloat16)
                 for p in ("re", "im"))


def from_device(o) -> np.ndarray:
    """Device output (complex64 tensor or bf16 plane pair) -> complex128 numpy array."""
    import torch
    if isinstance(o, (tuple, list)):
        re, im = (t.view(torch.int16).cpu().numpy().view(np.uint16) for t in o)
        return bf16_bits_to_f64(re) + 1j * bf16_bits_to_f64(im)
    return o.cpu().numpy().astype(np.complex128)


def sample_rows(B: int, H: int, T: int, n: int, seed: int = 0, tile: int = 256) -> np.ndarray:
    """(b, h, t) rows to check at full size: first/last rows, tile edges and random picks."""
    rng = np.random.default_rng(seed)
    ts = {0, 1, T - 1, T // 2}
    for e in range(tile, T, tile):
        ts.update({e - 1, e})
    ts = sorted(t for t in ts if 0 <= t < T)
    rows = []
    for i, t in enumerate(ts[: n // 2]):
        rows.append((int(rng.integers(B)), int(rng.integers(H)), t))
    while len(rows) < n:
        rows.append((int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(T))))
    return np.array(rows, dtype=np.int64)
