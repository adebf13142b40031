"""GPU parity of the backward: the HIP forward + backward against the fp64
backward oracle, on the same seeded inputs and incoming gradient, through the
C ABI.  The oracle recomputes its own forward from q, k, v; the HIP backward
takes O and the row denominators from the HIP forward, as a caller would.

Gradients are compared row by row (each query or key row of dQ, dK, dV).  A
row's scale is the larger of its reference values and of the terms the
computation subtracts to form it (`term_scales`): Born's dQ and dK are
differences X - Y of two sums (the delta = Re(G^H O) term, whose own terms
are counted by magnitude, sum_c |G_c| |O_c|, since delta is formed from the
forward's output as the caller stores it), and PCT's dq and dk remove a
projection.  Where X and Y cancel -- exactly so in Born's first
causal row, whose gradient is identically 0 because O[0] = V[0] -- fp32
arithmetic leaves rounding noise of the size of X and Y, which is what the
tolerance is measured against there.  (An fp32 emulation of the same
formulas on the CPU reproduces the kernel's error in such rows exactly.)
"""
import dataclasses
import math

import numpy as np
import pytest

from complex_valued_attention_amd import inputs as gen
from complex_valued_attention_amd.check import (GRAD_FLOOR, TOL, from_device, grad_to_device, rowwise_rel_err,
                                                to_device)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _cattn():
    from complex_valued_attention_amd import cattn
    cattn.lib()   # fail loudly if the HIP library is missing
    return cattn


def say(*a):
    print(*a, flush=True)


def run_hip_bwd(w, inp, grad, bias=0.0, eps=0.0):
    """(dq, dk, dv, db_rows or None) from the HIP forward + backward."""
    c = _cattn()
    q, k, v = to_device(inp)
    g = grad_to_device(grad)
    db = None
    if w.op == "born":
        den = torch.empty(w.B * w.H * w.T, dtype=torch.float32, device="cuda")
        o = c.born_fwd(q, k, v, causal=w.causal, eps=eps, row_den=den)
        dq, dk, dv = c.born_bwd(q, k, v, o, g, den, causal=w.causal)
    else:
        db = torch.full((w.B * w.H * w.T,), float("nan"), dtype=torch.float32, device="cuda")
        dq, dk, dv = c.pct_bwd(q, k, v, g, causal=w.causal, bias=bias, db_rows=db)
    torch.cuda.synchronize()
    return (from_device(dq), from_device(dk), from_device(dv),
            None if db is None else db.cpu().numpy().astype(np.float64))


def run_oracle_bwd(w, inp, grad, bias=0.0, eps=0.0, heads=None):
    import oracle
    q, k, v, g = inp.q64, inp.k64, inp.v64, grad.g64
    if heads is not None:   # (b, h) pairs: heads are independent
        sel = lambda x: np.stack([x[b, h] for b, h in heads])
        q, k, v, g = sel(q), sel(k), sel(v), sel(g)
    if w.op == "born":
        return oracle.born_attention_bwd(q, k, v, g, causal=w.causal, eps=eps) + (None,)
    return oracle.pct_attention_bwd(q, k, v, g, causal=w.causal, bias=bias)


def term_scales(op, q, k, v, g, causal, bias=0.0, eps=0.0, decay=None):
    """Per-row magnitude (max modulus) of the terms each gradient row is formed from,
    before they cancel: (dq, dk, dv) arrays of shape [..., T].  decay: per-head
    gammas [H] of q's head axis (Born, causal)."""
    T, d = q.shape[-2], q.shape[-1]
    mask = np.tril(np.ones((T, T))) if causal else np.ones((T, T))
    if decay is not None:
        dist = np.arange(T)[:, None] - np.arange(T)[None, :]
        gam = np.asarray(decay, dtype=np.float64)[:, None, None]
        mask = np.where(dist >= 0, gam ** np.maximum(dist, 0), 0.0)     # [H, T, T]
    tr = lambda x: np.swapaxes(x, -1, -2)
    amax = lambda x: np.abs(x).max(axis=-1)
    E = (g.conj() @ tr(v)).real * mask
    if op == "born":
        S = q @ tr(k.conj())
        wgt = (S.real ** 2 + S.imag ** 2) * mask
        l = wgt.sum(-1) + eps
        inv = np.where(l > 0, 1.0 / np.where(l > 0, l, 1.0), 0.0)
        o = (wgt * inv[..., None]).astype(np.complex128) @ v
        # delta = Re(G^H O) is itself a sum of cancelling terms, formed from the
        # forward's output as stored (bf16 planes for that layout); its terms'
        # magnitudes sum to sum_c |G_c| |O_c|, which is what O's rounding scales with
        delta_abs = np.sum(np.abs(g) * np.abs(o), -1)
        X = (2 * E * S * inv[..., None]) * mask
        Y = (2 * delta_abs[..., None] * S * inv[..., None]) * mask
        sq = np.maximum(amax(X @ k), amax(Y @ k))
        sk = np.maximum(amax(tr(X.conj()) @ q), amax(tr(Y.conj()) @ q))
        sv = amax(tr(wgt * inv[..., None]).astype(np.complex128) @ g)
        return sq, sk, sv
    n = lambda x: np.sqrt(np.sum(np.abs(x) ** 2, -1, keepdims=True))
    nq, nk = n(q), n(k)
    qh = q / np.where(nq > 0, nq, 1.0)
    kh = k / np.where(nk > 0, nk, 1.0)
    s = np.sqrt(d) * (qh @ tr(kh.conj())).real
    wgt = 1.0 / (1.0 + np.exp(-(s + bias))) * mask
    ds = E * wgt * (1 - wgt)
    gq = np.sqrt(d) * ds.astype(np.complex128) @ kh
    gk = np.sqrt(d) * tr(ds).astype(np.complex128) @ qh
    pq = np.abs(np.sum((gq.conj() * qh).real, -1)) * amax(qh)
    pk = np.abs(np.sum((gk.conj() * kh).real, -1)) * amax(kh)
    rq = np.where(nq[..., 0] > 0, 1.0 / np.where(nq[..., 0] > 0, nq[..., 0], 1.0), 0.0)
    rk = np.where(nk[..., 0] > 0, 1.0 / np.where(nk[..., 0] > 0, nk[..., 0], 1.0), 0.0)
    return np.maximum(amax(gq), pq) * rq, np.maximum(amax(gk), pk) * rk, amax(tr(wgt).astype(np.complex128) @ g)


def grad_err(got, ref, terms):
    """max over rows of max |got - ref| / max(|ref row|, term scale, GRAD_FLOOR * largest row)."""
    got = np.asarray(got).reshape(-1, ref.shape[-1])
    ref = np.asarray(ref).reshape(-1, ref.shape[-1])
    diff = np.abs(got - ref).max(-1)
    if not np.all(np.isfinite(diff)):
        return float("inf")
    scale = np.maximum(np.abs(ref).max(-1), np.asarray(terms).reshape(-1))
    scale = np.maximum(scale, GRAD_FLOOR * scale.max())
    ok = scale > 0
    if np.any(~ok & (diff > 0)):
        return float("inf")
    return float((diff[ok] / scale[ok]).max()) if ok.any() else 0.0


def compare(w, got, ref, tag, terms):
    tol = TOL[w.layout]
    errs = [grad_err(a, b, t) for a, b, t in zip(got[:3], ref[:3], terms)]
    plain = [rowwise_rel_err(a, b, floor=GRAD_FLOOR) for a, b in zip(got[:3], ref[:3])]
    say(f"{tag}: plain row-wise dq {plain[0]:.2e} dk {plain[1]:.2e} dv {plain[2]:.2e}")
    say(f"{tag}: dq {errs[0]:.3e} dk {errs[1]:.3e} dv {errs[2]:.3e} (tol {tol})")
    assert max(errs) <= tol, errs
    if ref[3] is not None:
        db_err = np.abs(got[3].reshape(ref[3].shape) - ref[3]).max() / max(np.abs(ref[3]).max(), 1e-30)
        say(f"{tag}: db_rows {db_err:.3e}")
        assert db_err <= tol


CASES = [
    # (op, layout, causal, B, H, T, d, qk_unit+rotary)
    ("born", "c64", True, 1, 2, 100, 64, True),
    ("born", "c64", False, 2, 1, 77, 16, False),
    ("born", "c64", True, 1, 1, 1, 64, False),
    ("born", "c64", True, 1, 1, 300, 128, False),
    ("born", "c64", True, 1, 2, 129, 1, False),
    ("born", "c64", True, 1, 1, 100, 3, False),
    ("born", "c64", True, 2, 2, 257, 32, True),
    ("born", "bf16", True, 1, 2, 300, 64, True),
    ("born", "bf16", False, 1, 1, 200, 16, False),
    ("born", "bf16", True, 1, 1, 150, 128, True),
    # the bf16 head-width-64 matrix-core path: causal and not, T = 1, tile edges,
    # B*H a multiple of 8 and not
    ("born", "bf16", False, 2, 1, 333, 64, True),
    ("born", "bf16", True, 1, 1, 1, 64, True),
    ("born", "bf16", True, 1, 3, 64, 64, True),
    ("born", "bf16", True, 2, 4, 129, 64, True),
    ("born", "bf16", True, 1, 8, 520, 64, False),
    ("born", "bf16", False, 1, 1, 127, 64, False),
    # tile multiples: the key-side kernel runs every stage (non-causal) or every
    # stage past the diagonal (causal) in its branch-free loop
    ("born", "bf16", False, 1, 2, 256, 64, True),
    ("born", "bf16", True, 1, 2, 384, 64, True),
    ("pct", "c64", True, 1, 2, 300, 64, False),
    ("pct", "c64", False, 1, 2, 65, 16, False),
    ("pct", "c64", True, 1, 1, 100, 17, False),
    ("pct", "bf16", True, 1, 2, 200, 64, False),
    ("pct", "c64", False, 1, 1, 300, 128, False),
    ("pct", "c64", True, 1, 1, 1, 64, False),
    # complex64 at widths 16/32/64 runs on the fp32 matrix cores: several
    # 128-row blocks, ragged tails, 8 heads (the XCD-grouped block order)
    ("born", "c64", True, 1, 2, 300, 64, True),
    ("born", "c64", False, 1, 3, 260, 32, False),
    ("born", "c64", True, 2, 4, 200, 16, False),
    ("pct", "c64", True, 2, 1, 520, 32, False),
    ("pct", "c64", False, 1, 8, 190, 64, False),
    ("pct", "c64", True, 1, 8, 300, 16, False),
    # bf16 planes on the fp32 matrix-core pair (widened on load): PCT at widths
    # 16/32/64 and Born at 16/32, causal and not, ragged tails, 8 heads
    ("pct", "bf16", False, 1, 2, 300, 64, False),
    ("pct", "bf16", True, 1, 8, 260, 32, False),
    ("pct", "bf16", True, 2, 1, 130, 16, False),
    ("born", "bf16", True, 1, 8, 200, 32, True),
    ("born", "bf16", False, 1, 3, 150, 32, False),
    # width 128 on the 16 x 16 fp32 matrix-core kernels: several 64-row blocks,
    # ragged tails, T below one 16-row tile, 8 heads, bf16 planes widened
    ("born", "c64", False, 1, 2, 200, 128, False),
    ("born", "c64", True, 1, 8, 260, 128, True),
    ("born", "c64", True, 2, 1, 16, 128, False),
    ("born", "c64", True, 1, 1, 9, 128, True),
    ("born", "bf16", False, 1, 1, 77, 128, False),
    ("born", "bf16", True, 2, 4, 192, 128, True),
    ("pct", "c64", True, 2, 4, 130, 128, False),
    ("pct", "c64", False, 1, 1, 1, 128, False),
    ("pct", "bf16", True, 1, 2, 150, 128, False),
    ("pct", "bf16", False, 1, 3, 64, 128, False),
]


@pytest.mark.parametrize("op,layout,causal,B,H,T,d,unit", CASES)
def test_bwd_parity(op, layout, causal, B, H, T, d, unit):
    w = gen.Workload("bwd", op, causal, B, H, T, d, layout, seed=21, qk_unit=unit, rotary=unit)
    say("case bwd", w)
    inp = gen.make_inputs(w)
    grad = gen.make_grad(w)
    bias = -math.log(T) if op == "pct" and T > 1 else 0.0
    got = run_hip_bwd(w, inp, grad, bias=bias)
    ref = run_oracle_bwd(w, inp, grad, bias=bias)
    terms = term_scales(op, inp.q64, inp.k64, inp.v64, grad.g64, causal, bias=bias)
    compare(w, got, ref, f"bwd {op} {layout} causal={causal} B{B} H{H} T{T} d{d}", terms)


@pytest.mark.parametrize("layout", ["c64", "bf16"])
def test_born_bwd_with_eps(layout):
    w = gen.Workload("bwd_eps", "born", True, 1, 2, 300, 64, layout, seed=22, qk_unit=True)
    inp = gen.make_inputs(w)
    grad = gen.make_grad(w)
    got = run_hip_bwd(w, inp, grad, eps=0.5)
    ref = run_oracle_bwd(w, inp, grad, eps=0.5)
    terms = term_scales("born", inp.q64, inp.k64, inp.v64, grad.g64, True, eps=0.5)
    compare(w, got, ref, f"bwd born eps=0.5 {layout}", terms)


# Full workload sizes in the launch configuration of a training step; the
# oracle checks whole heads (heads are independent).
FULL = [
    ("born_causal_c64_b4h8t1024d64_rotary", [(0, 0), (3, 7)]),
    ("pct_full_c64_b8h8t2048d64", [(5, 2)]),
    ("born_causal_bf16_b8h16t4096d64_rotary", [(7, 15)]),
]


# Width 128 at the B4 H8 T1024 shape (the complex64 rotary workload's shape)
# on the 16 x 16 fp32 matrix-core kernels, and bf16 planes at B2 H8 T2048.
FULL128 = [
    (gen.Workload("bwd128_c64", "born", True, 4, 8, 1024, 128, "c64", seed=24, qk_unit=True, rotary=True),
     [(0, 0), (3, 7)]),
    (gen.Workload("bwd128_pct", "pct", False, 4, 8, 1024, 128, "c64", seed=25), [(1, 3)]),
    (gen.Workload("bwd128_bf16", "born", True, 2, 8, 2048, 128, "bf16", seed=26, qk_unit=True, rotary=True),
     [(1, 7)]),
]


@pytest.mark.parametrize("w,heads", FULL128, ids=[f[0].name for f in FULL128])
def test_bwd_width128_sampled_heads(w, heads):
    say("case bwd 128", w)
    inp = gen.make_inputs(w)
    grad = gen.make_grad(w)
    bias = -math.log(w.T) if w.op == "pct" else 0.0
    got = run_hip_bwd(w, inp, grad, bias=bias)
    for x in got[:3]:
        assert np.isfinite(x).all()
    ref = run_oracle_bwd(w, inp, grad, bias=bias, heads=heads)
    sel = lambda x: np.stack([x[b, h] for b, h in heads])
    db = None if got[3] is None else sel(got[3].reshape(w.B, w.H, w.T))
    terms = term_scales(w.op, sel(inp.q64), sel(inp.k64), sel(inp.v64), sel(grad.g64), w.causal, bias=bias)
    compare(w, tuple(sel(x) for x in got[:3]) + (db,), ref, f"bwd 128 {w.name} heads {heads}", terms)


@pytest.mark.parametrize("name,heads", FULL, ids=[f[0] for f in FULL])
def test_bwd_full_size_sampled_heads(name, heads):
    w = gen.WORKLOADS[name]
    say("case bwd full", w)
    inp = gen.make_inputs(w)
    grad = gen.make_grad(w)
    got = run_hip_bwd(w, inp, grad)
    for x in got[:3]:
        assert np.isfinite(x).all()
    ref = run_oracle_bwd(w, inp, grad, heads=heads)
    sel = lambda x: np.stack([x[b, h] for b, h in heads])
    db = None if got[3] is None else sel(got[3].reshape(w.B, w.H, w.T))
    terms = term_scales(w.op, sel(inp.q64), sel(inp.k64), sel(inp.v64), sel(grad.g64), w.causal)
    compare(w, tuple(sel(x) for x in got[:3]) + (db,), ref, f"bwd full {name} heads {heads}", terms)


@pytest.mark.parametrize("op,d", [("born", 64), ("pct", 64), ("born", 128), ("pct", 128)])
def test_bwd_bitwise_deterministic(op, d):
    w = gen.Workload("det", op, True, 1, 2, 333, d, "c64", seed=23, qk_unit=True)
    inp = gen.make_inputs(w)
    grad = gen.make_grad(w)
    a = run_hip_bwd(w, inp, grad)
    b = run_hip_bwd(w, inp, grad)
    for x, y in zip(a[:3], b[:3]):
        assert np.array_equal(x, y)
