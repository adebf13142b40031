"""GPU parity at the operators' degenerate rows, on the matrix-core paths and
the element-wise one, forward and backward.

* PCT with zero-norm query or key rows: the inverse norm is 0, so every score
  touching such a row is 0 and its weight is the gate at 0 -- sigmoid(bias),
  exp(0) under the softmax cell, r^2 relu(-t)^2 under the screening cell.
* Born with zero query rows among live rows: every weight of that row is 0, so
  the row's denominator is eps, its output 0 (with eps = 0 the row is dead and
  written as 0 as well); the other rows are unaffected.  Zero key rows take no
  weight; a first query whose only key is zero is a dead row.
* The backward of both: a dead Born row contributes nothing, a zero-norm PCT
  row gets gradient 0.

Every case is compared with the fp64 oracle, which defines all of these rows.
"""
import math

import numpy as np
import pytest

from complex_valued_attention_amd import inputs as gen
from complex_valued_attention_amd.check import TOL, from_device, rowwise_rel_err, to_device

from test_gpu_bwd import compare, run_hip_bwd, run_oracle_bwd, term_scales

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _cattn():
    from complex_valued_attention_amd import cattn
    cattn.lib()   # fail loudly if the HIP library is missing
    return cattn


def say(*a):
    print(*a, flush=True)


def zero_rows(inp, name, rows):
    """Set rows (b, h, t) of operand `name` to exactly 0 in both the uploaded
    arrays and the oracle's copy."""
    x64 = getattr(inp, name + "64")
    for b, h, t in rows:
        x64[b, h, t] = 0
        if inp.layout == "c64":
            inp.dev[name][b, h, t] = 0
        else:
            inp.dev[name + "_re"][b, h, t] = 0
            inp.dev[name + "_im"][b, h, t] = 0


def pick_rows(B, H, T, ts):
    return [(b, h, t) for b in range(B) for h in range(H) for t in ts if t < T and (b + h + t) % 2 == 0] + \
        [(B - 1, H - 1, t) for t in ts if t < T]


ZT = [0, 5, 31, 32, 33, 127, 128, 200, 255, 256, 299]


def forward(c, op, q, k, v, causal, gate, a, b, eps=0.0, row_den=None):
    if op == "born":
        return c.born_fwd(q, k, v, causal=causal, eps=eps, row_den=row_den)
    return c.pct_gate_fwd(q, k, v, gate=gate, causal=causal, a=a, b=b)


def oracle_fwd(op, inp, causal, gate, a, b, eps=0.0):
    import oracle
    if op == "born":
        return oracle.born_attention(inp.q64, inp.k64, inp.v64, causal=causal, eps=eps, return_den=True)
    if gate == "sigmoid":
        return oracle.pct_attention(inp.q64, inp.k64, inp.v64, causal=causal, bias=a), None
    if gate == "softmax":
        return oracle.pct_softmax_attention(inp.q64, inp.k64, inp.v64, causal=causal), None
    return oracle.pct_screen_attention(inp.q64, inp.k64, inp.v64, causal=causal, r=a, t=b), None


PCT_CASES = [
    # (layout, causal, d, gate)
    ("c64", True, 64, "sigmoid"), ("c64", False, 64, "sigmoid"), ("bf16", True, 64, "sigmoid"),
    ("bf16", False, 32, "sigmoid"), ("c64", True, 16, "softmax"), ("bf16", False, 64, "softmax"),
    ("c64", False, 64, "screen"), ("bf16", True, 64, "screen"), ("c64", True, 17, "sigmoid"),
    ("bf16", True, 17, "softmax"),
]


@pytest.mark.parametrize("layout,causal,d,gate", PCT_CASES)
def test_pct_zero_query_and_key_rows(layout, causal, d, gate):
    c = _cattn()
    B, H, T = 1, 3, 300
    w = gen.Workload("edge_pct", "pct", causal, B, H, T, d, layout, seed=31)
    say("case pct zero rows", w, gate)
    inp = gen.make_inputs(w)
    zero_rows(inp, "q", pick_rows(B, H, T, ZT))
    zero_rows(inp, "k", pick_rows(B, H, T, [1, 6, 32, 64, 129, 254, 298]))
    # gate parameters: the sigmoid bias at the pages' -log N; a screening
    # threshold below every score (|s| <= sqrt(d_h)), so the gate is the
    # well-conditioned polynomial r^2 (s - t)^2 and the zero rows' score 0
    # keeps weight r^2 t^2
    a, b = {"sigmoid": (-math.log(T), 0.0), "softmax": (0.0, 0.0),
            "screen": (1.25, -(math.sqrt(d) + 0.5))}[gate]
    q, k, v = to_device(inp)
    got = from_device(forward(c, "pct", q, k, v, causal, gate, a, b))
    torch.cuda.synchronize()
    ref, _ = oracle_fwd("pct", inp, causal, gate, a, b)
    err = rowwise_rel_err(got, ref)
    say(f"pct zero rows {layout} causal={causal} d{d} {gate}: rowwise rel err {err:.3e}")
    assert err <= TOL[layout]
    # a zero query row sees every key through the gate at 0
    zq = pick_rows(B, H, T, ZT)[0]
    assert np.abs(ref[zq]).max() > 0


BORN_CASES = [
    # (layout, causal, d, eps)
    ("c64", True, 64, 0.0), ("c64", True, 64, 0.25), ("c64", False, 64, 0.0),
    ("bf16", True, 64, 0.0), ("bf16", True, 64, 0.25), ("bf16", False, 64, 0.0),
    ("bf16", True, 16, 0.0), ("bf16", True, 32, 0.25), ("bf16", True, 128, 0.0),
    ("c64", True, 16, 0.0), ("c64", True, 32, 0.0), ("c64", True, 17, 0.0), ("bf16", True, 3, 0.25),
]


@pytest.mark.parametrize("layout,causal,d,eps", BORN_CASES)
def test_born_zero_query_rows(layout, causal, d, eps):
    c = _cattn()
    B, H, T = 1, 3, 300
    w = gen.Workload("edge_born", "born", causal, B, H, T, d, layout, seed=32, qk_unit=True, rotary=True)
    say("case born zero rows", w, eps)
    inp = gen.make_inputs(w)
    zq = pick_rows(B, H, T, ZT)
    zero_rows(inp, "q", zq)
    # head 1: its first key is zero too, so its query 0 (if live) has no weight at all
    zero_rows(inp, "k", [(0, 1, 0), (0, 1, 77), (0, 2, 150)])
    q, k, v = to_device(inp)
    den = torch.full((B * H * T,), float("nan"), dtype=torch.float32, device="cuda")
    got = from_device(forward(c, "born", q, k, v, causal, None, 0.0, 0.0, eps=eps, row_den=den))
    torch.cuda.synchronize()
    ref, rden = oracle_fwd("born", inp, causal, None, 0.0, 0.0, eps=eps)
    err = rowwise_rel_err(got, ref)
    say(f"born zero rows {layout} causal={causal} d{d} eps={eps}: rowwise rel err {err:.3e}")
    assert err <= TOL[layout]
    for r in zq:
        assert np.all(got[r] == 0)                         # exactly zero, not just small
    gd = den.cpu().numpy().reshape(B, H, T)
    for r in zq:
        assert gd[r] == np.float32(eps)                    # sum of zero weights, plus eps
    live = rden > 0
    rel = np.abs(gd - rden)[live] / rden[live]
    assert rel.max() <= (1e-4 if layout == "c64" else 2e-2)
    if causal:   # head 1, query 0: its only key is zero -> a dead row (O = 0)
        assert np.all(got[0, 1, 0] == 0)


BWD_CASES = [
    # (op, layout, causal, d) -- the bf16 width-64 pair, the fp32 matrix-core pairs, the vector pair
    ("born", "bf16", True, 64), ("born", "bf16", False, 64), ("born", "c64", True, 64),
    ("born", "bf16", True, 32), ("born", "c64", True, 17),
    ("pct", "c64", True, 64), ("pct", "bf16", False, 64), ("pct", "c64", False, 16), ("pct", "c64", True, 17),
    # width 128: the 16 x 16 fp32 matrix-core kernels
    ("born", "c64", True, 128), ("born", "bf16", False, 128), ("pct", "c64", True, 128), ("pct", "bf16", False, 128),
]


@pytest.mark.parametrize("op,layout,causal,d", BWD_CASES)
def test_bwd_zero_rows(op, layout, causal, d):
    B, H, T = 1, 2, 300
    w = gen.Workload("edge_bwd", op, causal, B, H, T, d, layout, seed=33, qk_unit=(op == "born"),
                     rotary=(op == "born"))
    say("case bwd zero rows", w)
    inp = gen.make_inputs(w)
    grad = gen.make_grad(w)
    zero_rows(inp, "q", pick_rows(B, H, T, ZT))
    if op == "pct":
        zero_rows(inp, "k", pick_rows(B, H, T, [1, 6, 32, 64, 129, 254, 298]))
    else:
        zero_rows(inp, "k", [(0, 1, 0), (0, 1, 77)])
    bias = -math.log(T) if op == "pct" else 0.0
    got = run_hip_bwd(w, inp, grad, bias=bias)
    ref = run_oracle_bwd(w, inp, grad, bias=bias)
    terms = term_scales(op, inp.q64, inp.k64, inp.v64, grad.g64, causal, bias=bias)
    compare(w, got, ref, f"bwd zero rows {op} {layout} causal={causal} d{d}", terms)
    # zero-norm PCT rows and dead Born rows: exactly zero query-side gradient
    for b, h, t in pick_rows(B, H, T, ZT):
        assert np.all(got[0][b, h, t] == 0), (b, h, t)
