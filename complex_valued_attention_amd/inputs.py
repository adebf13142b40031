"""Seeded synthetic inputs for the complex-valued attention forward.

This module only draws and rounds numbers; it holds none of the attention
arithmetic.  Both the fp64 oracle and the HIP path consume exactly the arrays
made here: the oracle reads the values *after* rounding to the device dtype
(promoted back to fp64), so a parity comparison measures kernel error only.

Recipe (the pages give no dataset for the attention forward, so these stand
in for the shapes the pages train at):

* ``numpy.random.Generator(PCG64(seed))`` draws six fp64 arrays of shape
  ``[B, H, T, d_h]`` in the order Re Q, Im Q, Re K, Im K, Re V, Im V, each
  N(0, 1/2), so that every component is circularly-symmetric complex normal
  CN(0, 1) ("The Quantum Shortcut", section 5.6, draws its complex vectors
  from a circularly symmetric complex normal distribution).
* Optionally each token vector (over its d_h complex components) of Q, K
  (and V) is scaled to unit Euclidean norm.
* Optionally Q and K are given the rotary phase ``x[t, m] *= exp(i t theta_m)``
  with ``theta_m = 10000 ** (-m / d_h)`` ("Show HN: CNET", RotaryEmbed:
  position as a complex phase rotation, base 10000).
* The arrays are rounded once to the device dtype: complex64, or bf16 real
  and imaginary planes (fp64 -> fp32 -> bf16, round-to-nearest-even each
  time).
"""
from __future__ import annotations

import dataclasses
import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "BENCH_WORKLOAD", "make_inputs", "make_grad", "random_qkv",
    "round_to_bf16_bits", "bf16_bits_to_f64", "attention_flops", "decay_gammas",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    """One forward-pass workload: operator, mask, shape, layout and input recipe."""
    name: str
    op: str            # "born" or "pct"
    causal: bool
    B: int
    H: int
    T: int
    d_h: int
    layout: str        # "c64" (interleaved complex64) or "bf16" (two bf16 planes)
    seed: int
    qk_unit: bool = False   # scale each Q, K token vector to unit norm
    v_unit: bool = False    # scale each V token vector to unit norm
    rotary: bool = False    # rotary phase on Q and K (after the unit scaling)

    @property
    def rows(self) -> int:
        return self.B * self.H * self.T


# The five workloads: Born causal at the tiny head width of the H-Transformer
# (d_h = 16), Born causal with rotary unit-norm Q/K at T = 1024, PCT full
# attention at the Needle length 2048, the bf16 Born workload at T = 4096
# (B 8, H 16, d_h 64) and PCT causal at the Path-X length 16384; then 32768-
# and 65536-token bf16 Born sequences for the carried-state (linear) form,
# and a 32768-token complex64 one for its fp32 matrix-core kernels.
WORKLOADS = {
    w.name: w for w in [
        Workload("born_causal_c64_b1h1t128d16", "born", True, 1, 1, 128, 16, "c64", seed=0),
        Workload("born_causal_c64_b4h8t1024d64_rotary", "born", True, 4, 8, 1024, 64, "c64",
                 seed=1, qk_unit=True, v_unit=True, rotary=True),
        Workload("pct_full_c64_b8h8t2048d64", "pct", False, 8, 8, 2048, 64, "c64", seed=2),
        Workload("born_causal_bf16_b8h16t4096d64_rotary", "born", True, 8, 16, 4096, 64, "bf16",
                 seed=3, qk_unit=True, rotary=True),
        Workload("pct_causal_c64_b1h8t16384d64", "pct", True, 1, 8, 16384, 64, "c64", seed=4),
        # a long sequence for the chunked (carried-state) form against the quadratic kernel
        Workload("born_causal_bf16_b1h16t32768d64_rotary", "born", True, 1, 16, 32768, 64, "bf16",
                 seed=5, qk_unit=True, rotary=True),
        Workload("born_causal_bf16_b1h16t65536d64_rotary", "born", True, 1, 16, 65536, 64, "bf16",
                 seed=6, qk_unit=True, rotary=True),
        Workload("born_causal_c64_b1h16t32768d64_rotary", "born", True, 1, 16, 32768, 64, "c64",
                 seed=7, qk_unit=True, rotary=True),
    ]
}
BENCH_WORKLOAD = "born_causal_bf16_b8h16t4096d64_rotary"


def decay_gammas(H: int) -> np.ndarray:
    """Per-head decay values for the decayed Born workloads: a fixed geometric
    schedule gamma_h = 1 - 2^-(5 + 8 h / (H - 1)), from 0.969 (a memory of
    ~32 tokens) on head 0 to 0.99988 (~8192 tokens) on the last head, so the
    heads span short to long ranges.  The pages fix no values."""
    if H <= 1:
        return np.array([1.0 - 2.0 ** -5])[:H]
    return 1.0 - 2.0 ** -(5.0 + 8.0 * np.arange(H) / (H - 1))


def attention_flops(T: int, d_h: int, causal: bool, heads: int = 1) -> float:
    """Nominal real flops: 8 T^2 d_h for S = Q K^H plus 4 T^2 d_h for W V, halved if causal."""
    f = 12.0 * T * T * d_h * heads
    return f / 2 if causal else f


# --------------------------------------------------------------------------- rounding

def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp64 -> fp32 (RNE) -> bf16 (RNE); returns the bf16 bit patterns as uint16."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    # round to nearest even on the low 16 bits (inputs here are finite)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------- drawing

def _unit_rows(z: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(z.real ** 2 + z.imag ** 2, axis=-1, keepdims=True))
    return z / n


def _rotary(z: np.ndarray) -> np.ndarray:
    T, d = z.shape[-2], z.shape[-1]
    theta = 10000.0 ** (-np.arange(d, dtype=np.float64) / d)
    ang = np.arange(T, dtype=np.float64)[:, None] * theta[None, :]
    return z * np.exp(1j * ang)


def random_qkv(B, H, T, d_h, seed, *, qk_unit=False, v_unit=False, rotary=False):
    """Draw fp64 complex Q, K, V of shape [B, H, T, d_h] by the recipe above."""
    rng = np.random.Generator(np.random.PCG64(seed))
    shape = (B, H, T, d_h)
    s = np.sqrt(0.5)
    parts = [rng.standard_normal(shape) * s for _ in range(6)]
    q = parts[0] + 1j * parts[1]
    k = parts[2] + 1j * parts[3]
    v = parts[4] + 1j * parts[5]
    del parts
    if qk_unit:
        q, k = _unit_rows(q), _unit_rows(k)
    if v_unit:
        v = _unit_rows(v)
    if rotary:
        q, k = _rotary(q), _rotary(k)
    return q, k, v


@dataclasses.dataclass
class Inputs:
    """Host arrays for one run.

    ``q64, k64, v64``: complex128, the device values promoted to fp64 (what the
    oracle reads).  ``dev``: what is uploaded -- for "c64" a dict of complex64
    arrays ``q, k, v``; for "bf16" a dict of uint16 bf16 bit planes
    ``q_re, q_im, k_re, ...``.
    """
    layout: str
    q64: np.ndarray
    k64: np.ndarray
    v64: np.ndarray
    dev: dict


def round_inputs(q, k, v, layout: str) -> Inputs:
    if layout == "c64":
        dev = {n: np.ascontiguousarray(a.astype(np.complex64)) for n, a in (("q", q), ("k", k), ("v", v))}
        r = {n: dev[n].astype(np.complex128) for n in dev}
        return Inputs(layout, r["q"], r["k"], r["v"], dev)
    if layout == "bf16":
        dev, r = {}, {}
        for n, a in (("q", q), ("k", k), ("v", v)):
            re, im = round_to_bf16_bits(a.real), round_to_bf16_bits(a.imag)
            dev[n + "_re"], dev[n + "_im"] = re, im
            r[n] = bf16_bits_to_f64(re) + 1j * bf16_bits_to_f64(im)
        return Inputs(layout, r["q"], r["k"], r["v"], dev)
    raise ValueError(f"unknown layout {layout!r}")


def make_inputs(w: Workload | str, **override) -> Inputs:
    """Inputs for a named workload; keyword overrides (B, H, T, seed, ...) shrink it for tests."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    if override:
        w = dataclasses.replace(w, **override)
    q, k, v = random_qkv(w.B, w.H, w.T, w.d_h, w.seed, qk_unit=w.qk_unit,
                         v_unit=w.v_unit, rotary=w.rotary)
    return round_inputs(q, k, v, w.layout)


@dataclasses.dataclass
class Grad:
    """An incoming gradient G = dL/d(conj O) for the backward: ``g64`` (complex128,
    the device values promoted) and ``dev`` (``g`` complex64, or ``g_re``/``g_im``
    bf16 bit planes)."""
    layout: str
    g64: np.ndarray
    dev: dict


def make_grad(w: Workload | str, **override) -> Grad:
    """CN(0, 1) incoming gradient of the workload's output shape, drawn from
    PCG64(seed + 1000) (a stream apart from the inputs') and rounded like them."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    if override:
        w = dataclasses.replace(w, **override)
    rng = np.random.Generator(np.random.PCG64(w.seed + 1000))
    shape = (w.B, w.H, w.T, w.d_h)
    g = (rng.standard_normal(shape) + 1j * rng.standard_normal(shape)) * np.sqrt(0.5)
    if w.layout == "c64":
        dev = {"g": np.ascontiguousarray(g.astype(np.complex64))}
        return Grad(w.layout, dev["g"].astype(np.complex128), dev)
    re, im = round_to_bf16_bits(g.real), round_to_bf16_bits(g.imag)
    return Grad(w.layout, bf16_bits_to_f64(re) + 1j * bf16_bits_to_f64(im), {"g_re": re, "g_im": im})
