"""GPU parity of the PCT family's sibling gates (the L2-softmax cell and the
screening gate, "Complex-valued Phase-Coherent Transformers", Appendix D.2)
against the fp64 oracle, through the C ABI, on the same seeded inputs."""
import dataclasses
import math

import numpy as np
import pytest

from complex_valued_attention_amd import inputs as gen
from complex_valued_attention_amd.check import TOL, from_device, rowwise_rel_err, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(*a):
    print(*a, flush=True)


def run_hip(w, inp, gate, a=0.0, b=0.0):
    from complex_valued_attention_amd import cattn
    cattn.lib()
    q, k, v = to_device(inp)
    o = cattn.pct_gate_fwd(q, k, v, gate=gate, causal=w.causal, a=a, b=b)
    torch.cuda.synchronize()
    return from_device(o)


def run_oracle(w, q, k, v, gate, a=0.0, b=0.0):
    import oracle
    if gate == "softmax":
        return oracle.pct_softmax_attention(q, k, v, causal=w.causal)
    if gate == "screen":
        return oracle.pct_screen_attention(q, k, v, causal=w.causal, r=a, t=b)
    return oracle.pct_attention(q, k, v, causal=w.causal, bias=a)


CASES = [
    # (gate, layout, causal, B, H, T, d, a, b)
    ("softmax", "c64", True, 1, 2, 300, 64, 0.0, 0.0),
    ("softmax", "c64", False, 2, 1, 77, 16, 0.0, 0.0),
    ("softmax", "c64", True, 1, 2, 129, 32, 0.0, 0.0),
    ("softmax", "c64", True, 1, 1, 1, 64, 0.0, 0.0),
    ("softmax", "c64", True, 1, 1, 100, 17, 0.0, 0.0),
    ("softmax", "c64", False, 1, 1, 300, 128, 0.0, 0.0),
    ("softmax", "bf16", True, 1, 2, 200, 64, 0.0, 0.0),
    ("screen", "c64", True, 1, 2, 300, 64, 1.3, 0.5),
    ("screen", "c64", False, 2, 1, 77, 16, 0.7, -0.2),
    ("screen", "c64", True, 1, 1, 130, 32, 2.0, 1.5),
    ("screen", "c64", True, 1, 1, 100, 3, 1.0, 0.0),
    ("screen", "bf16", False, 1, 2, 200, 64, 1.0, 0.25),
    ("screen", "c64", True, 1, 1, 300, 128, 0.5, -1.0),
    ("sigmoid", "c64", True, 1, 2, 300, 64, -math.log(300), 0.0),
]


def screen_row_condition(w, inp, r, t):
    """Relative condition number of each output row of the screening gate
    w = r^2 relu(s - t)^2 with respect to relative errors in its scores:

        kappa_row = sum_j |dw_j/ds_j| |s_j| |v_j| / max_c |O_row|,
        dw/ds = 2 r^2 max(s - t, 0).

    A row whose output comes from one key just above the threshold has
    kappa = 2 s / (s - t), without bound as s comes down to t: fp32 scores
    (relative error of a few units of 2^-24) then cannot give a fixed relative
    accuracy whatever the order of summation.  Rows that share their weight
    among keys well clear of t have kappa of order 1 to 10.
    """
    import oracle
    s = oracle.pct_scores(inp.q64, inp.k64)
    x = np.maximum(s - t, 0.0)
    sens = 2 * r * r * x * np.abs(s)
    if w.causal:
        sens = sens * np.tril(np.ones((w.T, w.T)))
    vmax = np.abs(inp.v64).max(axis=-1)                      # [B, H, T] per key
    ref = oracle.pct_screen_attention(inp.q64, inp.k64, inp.v64, causal=w.causal, r=r, t=t)
    num = np.einsum("bhij,bhj->bhi", sens, vmax)
    den = np.abs(ref).max(axis=-1)
    return np.where(num > 0, num / np.maximum(den, 1e-300), 0.0)


KAPPA0 = 10.0   # the condition number up to which a row is held to the plain bar


@pytest.mark.parametrize("gate,layout,causal,B,H,T,d,a,b", CASES)
def test_gate_parity(gate, layout, causal, B, H, T, d, a, b):
    w = gen.Workload("gate", "pct", causal, B, H, T, d, layout, seed=41)
    say("case gate", gate, w, a, b)
    inp = gen.make_inputs(w)
    got = run_hip(w, inp, gate, a, b)
    ref = run_oracle(w, inp.q64, inp.k64, inp.v64, gate, a, b)
    err = rowwise_rel_err(got, ref)
    say(f"gate {gate} {layout} causal={causal} B{B} H{H} T{T} d{d}: {err:.3e} (tol {TOL[layout]})")
    if gate != "screen":
        assert err <= TOL[layout]
        return
    # screening gate: the row bar, scaled up only for rows whose condition
    # number exceeds KAPPA0 (an active key just above the threshold)
    kappa = screen_row_condition(w, inp, a, b)
    bar = TOL[layout] * np.maximum(1.0, kappa / KAPPA0)
    rowerr = np.abs(got - ref).max(axis=-1) / np.maximum(np.abs(ref).max(axis=-1), 1e-300)
    rowerr = np.where(np.abs(ref).max(axis=-1) > 0, rowerr, np.abs(got).max(axis=-1))
    say(f"  screen: rows above kappa {KAPPA0:g}: {int((kappa > KAPPA0).sum())} of {kappa.size}; "
        f"worst error / bar = {float((rowerr / bar).max()):.3f}")
    assert np.all(rowerr <= bar)


def test_screen_threshold_above_bound_gives_zero():
    w = gen.Workload("gate0", "pct", True, 1, 1, 200, 64, "c64", seed=42)
    inp = gen.make_inputs(w)
    got = run_hip(w, inp, "screen", 3.0, 8.0)   # t = sqrt(64): every weight is 0
    assert np.all(got == 0)


@pytest.mark.parametrize("name,gate,a,b", [("pct_full_c64_b8h8t2048d64", "softmax", 0.0, 0.0),
                                          ("pct_full_c64_b8h8t2048d64", "screen", 1.0, 0.5),
                                          ("pct_causal_c64_b1h8t16384d64", "softmax", 0.0, 0.0)])
def test_gate_full_size_whole_heads(name, gate, a, b):
    w = gen.WORKLOADS[name]
    say("case gate full", gate, w)
    inp = gen.make_inputs(w)
    got = run_hip(w, inp, gate, a, b)
    assert np.isfinite(got).all()
    heads = [(w.B - 1, w.H - 1)] if w.T > 4096 else [(0, 0), (w.B - 1, w.H - 1)]
    for bb, hh in heads:
        if w.T > 4096:   # one head of T = 16384: check sampled rows, each from its own prefix
            rows = [0, 1, 4095, 4096, 8191, w.T - 1]
            for t in rows:
                J = t + 1 if w.causal else w.T
                ref = run_oracle(w, inp.q64[bb, hh, t:t + 1], inp.k64[bb, hh, :J], inp.v64[bb, hh, :J],
                                 gate, a, b) if not w.causal else \
                    run_oracle(dataclasses.replace(w, causal=False), inp.q64[bb, hh, t:t + 1],
                               inp.k64[bb, hh, :J], inp.v64[bb, hh, :J], gate, a, b)
                err = rowwise_rel_err(got[bb, hh, t:t + 1], ref)
                assert err <= TOL[w.layout], (t, err)
            say(f"gate {gate} full {name} head {(bb, hh)} rows {rows}: ok")
        else:
            ref = run_oracle(w, inp.q64[bb, hh], inp.k64[bb, hh], inp.v64[bb, hh], gate, a, b)
            err = rowwise_rel_err(got[bb, hh], ref)
            say(f"gate {gate} full {name} head {(bb, hh)}: {err:.3e}")
            assert err <= TOL[w.layout]


@pytest.mark.parametrize("gate", ["softmax", "screen"])
def test_gate_bitwise_deterministic(gate):
    w = gen.Workload("gdet", "pct", True, 1, 2, 333, 64, "c64", seed=43)
    inp = gen.make_inputs(w)
    a = run_hip(w, inp, gate, 1.0, 0.1)
    b = run_hip(w, inp, gate, 1.0, 0.1)
    assert np.array_equal(a, b)
