"""GPU parity of the Born options against the fp64 oracle, through the C ABI:

* per-head decay (w = gamma_h^(k-j) |S|^2, causal) in the forward at small
  sizes on every kernel class, with eps and row denominators, and on sampled
  rows at the full shapes of the Born and PCT workloads (B4 H8 T1024,
  B8 H16 T4096 bf16, B1 H8 T16384);
* the carried state under decay: state build (overwrite and accumulate),
  prefill with a carried state and merge, token-by-token steps;
* the backward under decay;
* Q rotated at load (rotary_base) against the oracle's rotary + Born, and
  bitwise against the rotary pass followed by the plain forward.

The decay values go to the library as float32; the oracle uses the same
float32 values.
"""
import dataclasses

import numpy as np
import pytest

from complex_valued_attention_amd import inputs as gen
from complex_valued_attention_amd.check import TOL, from_device, rowwise_rel_err, sample_rows, to_device

from test_gpu_linear import DEN_TOL, _slice, _state_err, state_tol

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _cattn():
    from complex_valued_attention_amd import cattn
    cattn.lib()   # fail loudly if the HIP library is missing
    return cattn


def say(*a):
    print(*a, flush=True)


def f32(x):
    return np.asarray(x, dtype=np.float32).astype(np.float64)


FWD_CASES = [
    # (layout, B, H, T, d, gammas, eps)
    ("c64", 1, 3, 300, 64, (0.5, 0.97, 1.0), 0.0),
    ("bf16", 1, 3, 300, 64, (0.5, 0.97, 1.0), 0.0),
    ("bf16", 2, 3, 1000, 64, (0.8, 0.99, 0.9999), 0.1),
    ("c64", 2, 2, 700, 64, (0.9, 0.999), 0.0),
    ("c64", 1, 3, 128, 16, (0.5, 0.9, 0.999), 0.0),
    ("c64", 1, 2, 300, 32, (0.7, 0.995), 0.05),
    ("c64", 1, 2, 300, 17, (0.6, 0.99), 0.0),
    ("bf16", 1, 2, 257, 32, (0.75, 0.98), 0.0),
    ("bf16", 1, 2, 257, 16, (0.75, 0.98), 0.0),
    ("bf16", 1, 1, 300, 128, (0.95,), 0.0),
    ("c64", 1, 1, 300, 128, (0.95,), 0.0),
    ("bf16", 1, 2, 100, 3, (0.5, 0.9), 0.25),
    ("c64", 1, 2, 1, 64, (0.5, 0.9), 0.0),
    ("bf16", 1, 2, 65, 64, (1e-3, 0.5), 0.0),      # strong decay: far weights underflow
]


@pytest.mark.parametrize("layout,B,H,T,d,gammas,eps", FWD_CASES)
def test_decay_forward_small(layout, B, H, T, d, gammas, eps):
    import oracle
    c = _cattn()
    w = gen.Workload("decay", "born", True, B, H, T, d, layout, seed=91, qk_unit=True, rotary=True)
    say("case decay fwd", w, gammas, eps)
    inp = gen.make_inputs(w)
    q, k, v = to_device(inp)
    den = torch.full((B * H * T,), float("nan"), dtype=torch.float32, device="cuda")
    o = c.born_fwd(q, k, v, causal=True, eps=eps, row_den=den, decay=list(gammas))
    torch.cuda.synchronize()
    ref, rden = oracle.born_attention(inp.q64, inp.k64, inp.v64, causal=True, eps=eps, return_den=True,
                                      decay=f32(gammas))
    err = rowwise_rel_err(from_device(o), ref)
    gd = den.cpu().numpy().reshape(B, H, T).astype(np.float64)
    live = rden > 0
    den_err = float(np.max(np.abs(gd - rden)[live] / rden[live]))
    say(f"  rowwise rel err {err:.3e}, row_den {den_err:.3e}")
    assert err <= TOL[layout]
    assert den_err <= DEN_TOL[layout] * 2


@pytest.mark.parametrize("layout,d", [("c64", 64), ("bf16", 64), ("c64", 16), ("bf16", 32), ("bf16", 128),
                                      ("c64", 17)])
def test_decay_of_one_is_plain_born(layout, d):
    # every factor is exp2(0) = 1 exactly: the decayed instance must give the
    # plain kernel's bits
    import oracle
    c = _cattn()
    w = gen.Workload("decay1", "born", True, 1, 2, 300, d, layout, seed=92, qk_unit=True)
    inp = gen.make_inputs(w)
    q, k, v = to_device(inp)
    dd = torch.empty(2 * 300, dtype=torch.float32, device="cuda")
    dp = torch.empty(2 * 300, dtype=torch.float32, device="cuda")
    got = from_device(c.born_fwd(q, k, v, causal=True, decay=[1.0, 1.0], row_den=dd))
    plain = from_device(c.born_fwd(q, k, v, causal=True, row_den=dp))
    torch.cuda.synchronize()
    ref = oracle.born_attention(inp.q64, inp.k64, inp.v64, causal=True)
    err = rowwise_rel_err(got, ref)
    say(f"decay 1 {layout} d{d}: {err:.3e}, max |decay - plain| {np.abs(got - plain).max():.3e}")
    assert err <= TOL[layout]
    assert np.array_equal(got, plain)
    assert torch.equal(dd, dp)


FULL = {
    # the Born workloads' shapes and the PCT causal workload's shape, as Born with decay
    "c1": dataclasses.replace(gen.WORKLOADS["born_causal_c64_b4h8t1024d64_rotary"]),
    "c3": dataclasses.replace(gen.WORKLOADS["born_causal_bf16_b8h16t4096d64_rotary"]),
    "c4": dataclasses.replace(gen.WORKLOADS["pct_causal_c64_b1h8t16384d64"], op="born", qk_unit=True),
}


@pytest.mark.parametrize("key", list(FULL))
def test_decay_full_size_sampled(key):
    import oracle
    c = _cattn()
    w = FULL[key]
    gam = gen.decay_gammas(w.H)
    say("case decay full", key, w)
    inp = gen.make_inputs(w)
    q, k, v = to_device(inp)
    got = from_device(c.born_fwd(q, k, v, causal=True, decay=gam))
    torch.cuda.synchronize()
    assert np.isfinite(got).all()
    rows = sample_rows(w.B, w.H, w.T, 64, seed=w.seed)
    ref = oracle.born_attention_rows(inp.q64, inp.k64, inp.v64, rows, causal=True, decay=f32(gam))
    err = rowwise_rel_err(got[rows[:, 0], rows[:, 1], rows[:, 2]], ref)
    say(f"  {len(rows)} sampled rows: rowwise rel err {err:.3e}")
    assert err <= TOL[w.layout]


# ----------------------------------------------------------------------------- carried state

def _oracle_state_decay(inp, B, H, t0, t1, gam):
    import oracle
    d = inp.k64.shape[-1]
    S = np.zeros((B, H, 2 * d + 1, d, d))
    for b in range(B):
        for h in range(H):
            S[b, h] = oracle.pack_state(*oracle.born_state(inp.k64[b, h, t0:t1], inp.v64[b, h, t0:t1],
                                                           gamma=gam[h]))
    return S


LIN_CASES = [
    # (layout, B, H, T, T1, d, eps)
    ("c64", 1, 2, 300, 129, 64, 0.0),
    ("bf16", 1, 2, 300, 100, 64, 0.0),
    ("c64", 2, 2, 150, 17, 16, 0.25),
    ("bf16", 1, 2, 333, 100, 32, 0.0),
    ("c64", 1, 2, 200, 64, 33, 0.0),
    ("bf16", 2, 3, 700, 300, 64, 0.1),
]


@pytest.mark.parametrize("layout,B,H,T,T1,d,eps", LIN_CASES)
def test_decay_state_and_prefill(layout, B, H, T, T1, d, eps):
    import oracle
    c = _cattn()
    gam = f32(np.linspace(0.9, 0.999, H))
    w = gen.Workload("dcarry", "born", True, B, H, T, d, layout, seed=93, qk_unit=True)
    inp = gen.make_inputs(w)
    q, k, v = to_device(inp)
    say(f"decay carry {layout} B{B} H{H} T{T} split {T1} d{d} eps {eps}")
    # state build, overwrite then accumulate
    S = c.born_state_buffer(B, H, d)
    S.fill_(float("nan"))
    c.born_state(_slice(k, 0, T1), _slice(v, 0, T1), S, decay=gam)
    torch.cuda.synchronize()
    err = _state_err(S, _oracle_state_decay(inp, B, H, 0, T1, gam))
    say(f"  state of the first {T1} tokens: {err:.3e}")
    assert err <= state_tol(layout, d)
    # prefill of the rest with the carried state, then carry the rest out
    q2, k2, v2 = (_slice(x, T1, T) for x in (q, k, v))
    row_den = torch.empty(B * H * (T - T1), dtype=torch.float32, device="cuda")
    o2 = c.born_fwd(q2, k2, v2, causal=True, eps=eps, row_den=row_den, decay=gam)
    c.born_merge(q2, S, o2, row_den, decay=gam)
    c.born_state(k2, v2, S, accumulate=True, decay=gam)
    torch.cuda.synchronize()
    ref, rden = oracle.born_attention(inp.q64, inp.k64, inp.v64, causal=True, eps=eps, return_den=True, decay=gam)
    err = rowwise_rel_err(from_device(o2), ref[:, :, T1:])
    say(f"  merged output: {err:.3e}")
    assert err <= TOL[layout]
    l_got = row_den.cpu().numpy().reshape(B, H, T - T1)
    den_err = float(np.max(np.abs(l_got - rden[:, :, T1:]) / rden[:, :, T1:]))
    say(f"  merged row_den: {den_err:.3e}")
    assert den_err <= DEN_TOL[layout] * 2
    err = _state_err(S, _oracle_state_decay(inp, B, H, 0, T, gam))
    say(f"  state after accumulate: {err:.3e}")
    assert err <= state_tol(layout, d)


@pytest.mark.parametrize("layout,d", [("c64", 64), ("bf16", 64), ("c64", 20), ("bf16", 16)])
def test_decay_steps(layout, d):
    import oracle
    c = _cattn()
    B, H, T0, n, eps = 1, 2, 40, 12, 0.0
    gam = f32([0.8, 0.99])
    T = T0 + n
    w = gen.Workload("dstep", "born", True, B, H, T, d, layout, seed=94)
    inp = gen.make_inputs(w)
    q, k, v = to_device(inp)
    say(f"decay steps {layout} d{d}")
    S = c.born_state_buffer(B, H, d)
    c.born_state(_slice(k, 0, T0), _slice(v, 0, T0), S, decay=gam)
    outs = []
    for t in range(T0, T):
        o, _ = c.born_step(*(_slice(x, t, t + 1) for x in (q, k, v)), S, eps=eps, decay=gam)
        outs.append(from_device(o))
    torch.cuda.synchronize()
    got = np.concatenate(outs, axis=2)
    ref = oracle.born_attention(inp.q64, inp.k64, inp.v64, causal=True, eps=eps, decay=gam)[:, :, T0:]
    err = rowwise_rel_err(got, ref)
    say(f"  outputs: {err:.3e}")
    assert err <= TOL[layout]
    assert _state_err(S, _oracle_state_decay(inp, B, H, 0, T, gam)) <= state_tol(layout, d)


# ----------------------------------------------------------------------------- backward

BWD_CASES = [
    # (layout, B, H, T, d)
    ("bf16", 1, 2, 300, 64),
    ("c64", 1, 2, 300, 64),
    ("c64", 1, 2, 200, 16),
    ("c64", 1, 1, 150, 17),
    ("bf16", 1, 2, 257, 32),
    ("c64", 1, 2, 200, 128),
    ("bf16", 1, 8, 130, 128),
]


@pytest.mark.parametrize("layout,B,H,T,d", BWD_CASES)
def test_decay_backward(layout, B, H, T, d):
    import oracle
    from complex_valued_attention_amd.check import grad_to_device
    from test_gpu_bwd import compare, term_scales
    c = _cattn()
    gam = f32(np.linspace(0.7, 0.995, H))
    w = gen.Workload("dbwd", "born", True, B, H, T, d, layout, seed=95, qk_unit=True, rotary=True)
    say("case decay bwd", w)
    inp = gen.make_inputs(w)
    grad = gen.make_grad(w)
    q, k, v = to_device(inp)
    den = torch.empty(B * H * T, dtype=torch.float32, device="cuda")
    o = c.born_fwd(q, k, v, causal=True, row_den=den, decay=gam)
    dq, dk, dv = c.born_bwd(q, k, v, o, grad_to_device(grad), den, causal=True, decay=gam)
    torch.cuda.synchronize()
    got = tuple(from_device(x) for x in (dq, dk, dv)) + (None,)
    ref = tuple(oracle.born_attention_bwd(inp.q64, inp.k64, inp.v64, grad.g64, causal=True, decay=gam)) + (None,)
    terms = term_scales("born", inp.q64, inp.k64, inp.v64, grad.g64, True, decay=gam)
    compare(w, got, ref, f"decay bwd {layout} d{d}", terms)


@pytest.mark.parametrize("layout,d", [("bf16", 64), ("c64", 64), ("c64", 16), ("bf16", 32), ("c64", 17), ("c64", 128),
                                      ("bf16", 128)])
def test_decay_of_one_backward_is_plain(layout, d):
    # every factor is exp2(0) = 1 exactly: the decayed instances give the plain gradients' bits
    from complex_valued_attention_amd.check import grad_to_device
    c = _cattn()
    B, H, T = 1, 2, 300
    w = gen.Workload("dbwd1", "born", True, B, H, T, d, layout, seed=97, qk_unit=True)
    inp = gen.make_inputs(w)
    grad = gen.make_grad(w)
    q, k, v = to_device(inp)
    g = grad_to_device(grad)
    den = torch.empty(B * H * T, dtype=torch.float32, device="cuda")
    o = c.born_fwd(q, k, v, causal=True, row_den=den)
    a = c.born_bwd(q, k, v, o, g, den, causal=True, decay=[1.0] * H)
    b = c.born_bwd(q, k, v, o, g, den, causal=True)
    torch.cuda.synchronize()
    for name, x, y in zip(("dq", "dk", "dv"), a, b):
        xa, ya = from_device(x), from_device(y)
        say(f"decay 1 bwd {layout} d{d} {name}: max |diff| {np.abs(xa - ya).max():.3e}")
        assert np.array_equal(xa, ya), name


def test_decay_backward_full_size_heads():
    # the B8 H16 T4096 bf16 shape on the matrix-core pair, two whole heads against the oracle
    import oracle
    from complex_valued_attention_amd.check import grad_to_device
    from test_gpu_bwd import compare, term_scales
    c = _cattn()
    w = FULL["c3"]
    gam = gen.decay_gammas(w.H)
    say("case decay bwd full", w)
    inp = gen.make_inputs(w)
    grad = gen.make_grad(w)
    q, k, v = to_device(inp)
    den = torch.empty(w.B * w.H * w.T, dtype=torch.float32, device="cuda")
    o = c.born_fwd(q, k, v, causal=True, row_den=den, decay=gam)
    dq, dk, dv = c.born_bwd(q, k, v, o, grad_to_device(grad), den, causal=True, decay=gam)
    torch.cuda.synchronize()
    got = [from_device(x) for x in (dq, dk, dv)]
    g32 = f32(gam)
    for b, h in [(0, 0), (7, 15)]:
        ref = oracle.born_attention_bwd(inp.q64[b, h], inp.k64[b, h], inp.v64[b, h], grad.g64[b, h], causal=True,
                                        decay=g32[h])
        terms = term_scales("born", inp.q64[b, h][None], inp.k64[b, h][None], inp.v64[b, h][None],
                            grad.g64[b, h][None], True, decay=g32[h:h + 1])
        compare(w, tuple(x[b, h] for x in got) + (None,), tuple(ref) + (None,), f"decay bwd full head {b},{h}",
                tuple(t[0] for t in terms))


# ----------------------------------------------------------------------------- rotary Q at load

ROT_CASES = [
    # (layout, B, H, T, d, pos0)
    ("c64", 1, 2, 300, 64, 0),
    ("bf16", 1, 2, 300, 64, 0),
    ("bf16", 1, 2, 300, 64, 12345),
    ("c64", 1, 2, 200, 16, 7),
    ("c64", 1, 2, 100, 17, 0),
    ("bf16", 1, 2, 257, 32, 0),
    ("bf16", 1, 1, 100, 3, 99),
]


@pytest.mark.parametrize("layout,B,H,T,d,pos0", ROT_CASES)
def test_rotary_q_at_load(layout, B, H, T, d, pos0):
    import oracle
    c = _cattn()
    w = gen.Workload("rotq", "born", True, B, H, T, d, layout, seed=96, qk_unit=True)
    say("case rotary q", w, pos0)
    inp = gen.make_inputs(w)
    q, k, v = to_device(inp)
    # K is rotated by the rotary pass (as a key cache holds it); Q at load
    kr = c.rotary(k, pos0=pos0, base=10000.0)
    fused = c.born_fwd(q, kr, v, causal=True, rotary_base=10000.0, rotary_pos0=pos0)
    # the same through the rotary pass over Q
    qr = c.rotary(q, pos0=pos0, base=10000.0)
    plain = c.born_fwd(qr, kr, v, causal=True)
    torch.cuda.synchronize()
    # oracle: rotate both in fp64 from the rounded inputs
    q64 = oracle.rotary(inp.q64, pos0=pos0)
    k64 = oracle.rotary(inp.k64, pos0=pos0)
    ref = oracle.born_attention(q64, k64, inp.v64, causal=True)
    err = rowwise_rel_err(from_device(fused), ref)
    say(f"  fused vs oracle: {err:.3e}")
    assert err <= TOL[layout]
    a, b = from_device(fused), from_device(plain)
    say(f"  fused vs rotary pass + forward: max |diff| {np.abs(a - b).max():.3e}")
    assert np.array_equal(a, b)
