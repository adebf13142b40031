"""GPU parity: the HIP path against the fp64 oracle, element by element on the
same seeded inputs, through the C ABI.

Small cases run every output row (several tiles and a ragged tail); the full
workload sizes run in the launch configuration the benchmark times and are
checked on sampled rows the oracle computes one by one.
"""
import dataclasses
import math

import numpy as np
import pytest

from complex_valued_attention_amd import inputs as gen
from complex_valued_attention_amd.check import TOL, from_device, rowwise_rel_err, sample_rows, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _cattn():
    from complex_valued_attention_amd import cattn
    cattn.lib()   # fail loudly if the HIP library is missing
    return cattn


def run_hip(w: gen.Workload, inp: gen.Inputs, bias=0.0, eps=0.0, row_den=None):
    c = _cattn()
    q, k, v = to_device(inp)
    if w.op == "born":
        o = c.born_fwd(q, k, v, causal=w.causal, eps=eps, row_den=row_den)
    else:
        o = c.pct_fwd(q, k, v, causal=w.causal, bias=bias)
    torch.cuda.synchronize()
    return from_device(o)


def run_oracle(w, inp, bias=0.0, eps=0.0):
    import oracle
    if w.op == "born":
        return oracle.born_attention(inp.q64, inp.k64, inp.v64, causal=w.causal, eps=eps)
    return oracle.pct_attention(inp.q64, inp.k64, inp.v64, causal=w.causal, bias=bias)


def say(*a):
    print(*a, flush=True)


SMALL = []
for name, w in gen.WORKLOADS.items():
    for T in sorted({min(w.T, 128), 300, 1000}):
        SMALL.append(pytest.param(name, T, id=f"{name}-T{T}"))


@pytest.mark.parametrize("name,T", SMALL)
def test_parity_small(name, T):
    w = dataclasses.replace(gen.WORKLOADS[name], B=1, H=3, T=T)
    say("case", w)
    inp = gen.make_inputs(w)
    got = run_hip(w, inp)
    ref = run_oracle(w, inp)
    err = rowwise_rel_err(got, ref)
    say(f"{name} T={T} rowwise rel err {err:.3e} (tol {TOL[w.layout]})")
    assert err <= TOL[w.layout]


@pytest.mark.parametrize("name", list(gen.WORKLOADS))
def test_parity_full_size_sampled(name):
    import oracle
    w = gen.WORKLOADS[name]
    say("case full", w)
    inp = gen.make_inputs(w)
    got = run_hip(w, inp)
    assert np.isfinite(got).all()
    rows = sample_rows(w.B, w.H, w.T, 96, seed=w.seed)
    fn = oracle.born_attention_rows if w.op == "born" else oracle.pct_attention_rows
    ref = fn(inp.q64, inp.k64, inp.v64, rows, causal=w.causal)
    err = rowwise_rel_err(got[rows[:, 0], rows[:, 1], rows[:, 2]], ref)
    say(f"{name} full size, {len(rows)} sampled rows: rowwise rel err {err:.3e}")
    assert err <= TOL[w.layout]


@pytest.mark.parametrize("name", ["pct_full_c64_b8h8t2048d64", "pct_causal_c64_b1h8t16384d64"])
def test_pct_bf16_planes_full_size_sampled(name):
    # the PCT workloads' shapes on bf16 planes (the fp32 matrix-core kernel, widened on load)
    import oracle
    w = dataclasses.replace(gen.WORKLOADS[name], layout="bf16")
    say("case full bf16", w)
    inp = gen.make_inputs(w)
    got = run_hip(w, inp)
    assert np.isfinite(got).all()
    rows = sample_rows(w.B, w.H, w.T, 96, seed=w.seed)
    ref = oracle.pct_attention_rows(inp.q64, inp.k64, inp.v64, rows, causal=w.causal)
    err = rowwise_rel_err(got[rows[:, 0], rows[:, 1], rows[:, 2]], ref)
    say(f"{name} on bf16 planes, {len(rows)} sampled rows: rowwise rel err {err:.3e}")
    assert err <= TOL["bf16"]


EDGE = [
    # (op, layout, causal, B, H, T, d)
    ("born", "c64", True, 1, 1, 1, 64),
    ("born", "bf16", True, 1, 1, 1, 64),
    ("pct", "c64", True, 1, 1, 1, 64),
    ("born", "c64", False, 2, 1, 77, 64),
    ("born", "bf16", False, 1, 2, 333, 64),
    ("pct", "bf16", True, 1, 2, 200, 64),
    ("pct", "c64", False, 1, 2, 65, 16),
    ("born", "c64", True, 1, 2, 129, 1),
    ("born", "c64", True, 1, 1, 100, 3),
    ("pct", "c64", True, 1, 1, 100, 17),
    ("born", "bf16", True, 1, 2, 257, 16),
    ("born", "bf16", True, 1, 2, 257, 32),
    ("born", "bf16", True, 1, 1, 300, 128),
    ("born", "c64", True, 1, 1, 300, 128),
    ("pct", "c64", False, 1, 1, 300, 128),
    ("born", "c64", True, 3, 5, 33, 32),
]


@pytest.mark.parametrize("op,layout,causal,B,H,T,d", EDGE)
def test_parity_edge_shapes(op, layout, causal, B, H, T, d):
    w = gen.Workload("edge", op, causal, B, H, T, d, layout, seed=11, qk_unit=(op == "born"))
    say("case edge", w)
    inp = gen.make_inputs(w)
    got = run_hip(w, inp)
    ref = run_oracle(w, inp)
    err = rowwise_rel_err(got, ref)
    say(f"edge {op} {layout} causal={causal} B{B} H{H} T{T} d{d}: {err:.3e}")
    assert err <= TOL[layout]


# complex64 row-block pairs (64-query blocks, eight waves per pair) and the
# causal helpers: one block (helpers from the start), an odd block count (a
# middle block without a partner), even counts, ragged tails, every matrix
# width
# bf16 planes take the same kernel for the PCT cells (widened to fp32 on load)
PAIRS = [(op, causal, T, d, "c64") for op in ("born", "pct") for T in (64, 65, 191, 256, 449, 513)
         for d in (16, 32, 64, 128) for causal in (True,)] + \
        [(op, False, T, d, "c64") for op in ("born", "pct") for T in (65, 191, 513) for d in (16, 64, 128)] + \
        [("pct", causal, T, d, "bf16") for causal in (True, False) for T in (65, 191, 513)
         for d in (16, 32, 64, 128)]


@pytest.mark.parametrize("op,causal,T,d,layout", PAIRS)
def test_row_block_pairs_and_helpers(op, causal, T, d, layout):
    import oracle
    w = gen.Workload("pairs", op, causal, 1, 2, T, d, layout, seed=13)
    say("case", w)
    inp = gen.make_inputs(w)
    den = torch.full((2 * T,), float("nan"), dtype=torch.float32, device="cuda") if op == "born" else None
    got = run_hip(w, inp, row_den=den)
    ref = run_oracle(w, inp)
    err = rowwise_rel_err(got, ref)
    say(f"pairs {op} {layout} causal={causal} T={T} d={d}: rowwise rel err {err:.3e}")
    assert err <= TOL[layout]
    if op == "born":   # every row's denominator is written too
        _, ref_den = oracle.born_attention(inp.q64, inp.k64, inp.v64, causal=causal, return_den=True)
        np.testing.assert_allclose(den.cpu().numpy(), ref_den.reshape(-1), rtol=1e-4)


@pytest.mark.parametrize("layout", ["c64", "bf16"])
def test_born_eps_and_row_den(layout):
    import oracle
    w = gen.Workload("eps", "born", True, 1, 2, 300, 64, layout, seed=5, qk_unit=True)
    inp = gen.make_inputs(w)
    den = torch.full((2 * 300,), float("nan"), dtype=torch.float32, device="cuda")
    got = run_hip(w, inp, eps=0.5, row_den=den)
    ref, ref_den = oracle.born_attention(inp.q64, inp.k64, inp.v64, causal=True, eps=0.5, return_den=True)
    assert rowwise_rel_err(got, ref) <= TOL[layout]
    np.testing.assert_allclose(den.cpu().numpy(), ref_den.reshape(-1), rtol=1e-4 if layout == "c64" else 2e-2)


@pytest.mark.parametrize("layout", ["c64", "bf16"])
def test_pct_bias_minus_log_T(layout):
    T = 500
    w = gen.Workload("bias", "pct", True, 1, 2, T, 64, layout, seed=6)
    inp = gen.make_inputs(w)
    got = run_hip(w, inp, bias=-math.log(T))
    ref = run_oracle(w, inp, bias=-math.log(T))
    assert rowwise_rel_err(got, ref) <= TOL[layout]


@pytest.mark.parametrize("layout", ["c64", "bf16"])
def test_born_zero_keys_give_zero_rows(layout):
    w = gen.Workload("zk", "born", True, 1, 1, 130, 64, layout, seed=7)
    inp = gen.make_inputs(w)
    inp.k64[:] = 0
    for n in list(inp.dev):
        if n.startswith("k"):
            inp.dev[n][:] = 0
    got = run_hip(w, inp)
    assert np.all(got == 0)


# ----------------------------------------------------------------------------- properties on the kernel

@pytest.mark.parametrize("layout", ["c64", "bf16"])
def test_born_constant_values_rows_sum_to_one(layout):
    w = gen.Workload("const", "born", True, 2, 2, 700, 64, layout, seed=8, qk_unit=True, rotary=True)
    inp = gen.make_inputs(w)
    c = (0.6 - 0.3j) * np.ones(64)
    inp.v64[:] = c
    if layout == "c64":
        inp.dev["v"][:] = c.astype(np.complex64)
    else:
        inp.dev["v_re"][:] = gen.round_to_bf16_bits(np.full(64, 0.6))
        inp.dev["v_im"][:] = gen.round_to_bf16_bits(np.full(64, -0.3))
    got = run_hip(w, inp)
    tol = 1e-5 if layout == "c64" else 1e-2
    np.testing.assert_allclose(got, np.broadcast_to(c, got.shape), rtol=tol, atol=tol)


@pytest.mark.parametrize("layout", ["c64", "bf16"])
def test_born_first_row_is_v0_and_phase_invariance(layout):
    w = gen.Workload("ph", "born", True, 1, 2, 260, 64, layout, seed=9)
    inp = gen.make_inputs(w)
    base = run_hip(w, inp)
    np.testing.assert_allclose(base[:, :, 0], inp.v64[:, :, 0], rtol=0, atol=1e-6 if layout == "c64" else 1e-2)
    # multiply every token of Q and K by i (exact in both layouts): the output must not move
    rot = gen.Inputs(layout, inp.q64 * 1j, inp.k64 * 1j, inp.v64, {})
    if layout == "c64":
        rot.dev = {"q": (inp.dev["q"] * 1j).astype(np.complex64), "k": (inp.dev["k"] * 1j).astype(np.complex64),
                   "v": inp.dev["v"]}
    else:
        neg = lambda b: b ^ np.uint16(0x8000)
        rot.dev = {"q_re": neg(inp.dev["q_im"]), "q_im": inp.dev["q_re"], "k_re": neg(inp.dev["k_im"]),
                   "k_im": inp.dev["k_re"], "v_re": inp.dev["v_re"], "v_im": inp.dev["v_im"]}
    got = run_hip(w, rot)
    assert rowwise_rel_err(got, base) <= (1e-5 if layout == "c64" else 1e-2)


def test_pct_scale_invariance():
    w = gen.Workload("sc", "pct", False, 1, 2, 300, 64, "c64", seed=10)
    inp = gen.make_inputs(w)
    base = run_hip(w, inp)
    scaled = gen.Inputs("c64", inp.q64 * 8.0, inp.k64 * 0.125, inp.v64,
                        {"q": inp.dev["q"] * np.float32(8.0), "k": inp.dev["k"] * np.float32(0.125),
                         "v": inp.dev["v"]})
    got = run_hip(w, scaled)
    assert rowwise_rel_err(got, base) <= 1e-5


@pytest.mark.parametrize("name", ["born_causal_bf16_b8h16t4096d64_rotary", "pct_causal_c64_b1h8t16384d64"])
def test_head_slicing(name):
    # one call over [B, H] equals per-head calls
    w = dataclasses.replace(gen.WORKLOADS[name], B=2, H=3, T=520)
    inp = gen.make_inputs(w)
    full = run_hip(w, inp)
    for b in range(2):
        for h in range(3):
            sub = gen.Inputs(w.layout, inp.q64[b:b + 1, h:h + 1], inp.k64[b:b + 1, h:h + 1],
                             inp.v64[b:b + 1, h:h + 1],
                             {n: np.ascontiguousarray(a[b:b + 1, h:h + 1]) for n, a in inp.dev.items()})
            one = run_hip(dataclasses.replace(w, B=1, H=1), sub)
            assert np.array_equal(one[0, 0], full[b, h])


@pytest.mark.parametrize("name", list(gen.WORKLOADS))
def test_bitwise_deterministic_and_fully_written(name):
    c = _cattn()
    w = dataclasses.replace(gen.WORKLOADS[name], B=1, H=2, T=min(gen.WORKLOADS[name].T, 777))
    inp = gen.make_inputs(w)
    q, k, v = to_device(inp)
    outs = []
    for rep in range(3):
        if w.layout == "c64":
            o = torch.full(q.shape, float("nan"), dtype=torch.complex64, device="cuda")
        else:
            o = tuple(torch.full(q[0].shape, float("nan"), dtype=torch.bfloat16, device="cuda") for _ in range(2))
        if w.op == "born":
            c.born_fwd(q, k, v, causal=w.causal, out=o)
        else:
            c.pct_fwd(q, k, v, causal=w.causal, out=o)
        torch.cuda.synchronize()
        outs.append(from_device(o))
    assert np.isfinite(outs[0]).all()
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_side_stream_and_empty():
    c = _cattn()
    w = gen.Workload("st", "born", True, 1, 1, 200, 64, "bf16", seed=12, qk_unit=True)
    inp = gen.make_inputs(w)
    q, k, v = to_device(inp)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o = c.born_fwd(q, k, v)
    s.synchronize()
    ref = run_oracle(w, inp)
    assert rowwise_rel_err(from_device(o), ref) <= TOL["bf16"]
    e = torch.empty(1, 1, 0, 64, dtype=torch.complex64, device="cuda")
    out = c.born_fwd(e, e, e)
    assert out.shape == e.shape
