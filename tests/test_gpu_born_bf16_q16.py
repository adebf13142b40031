"""GPU parity of the Born forward on bf16 planes at head widths 128 and 32
(16-query tiles, 16 x 16 x 32 products) against the fp64 oracle, through the
C ABI.

Small cases cover every output row and denominator: one query, ragged tails
around the 16-query tile, the 32-key stage and the 128-query row block, odd
and even row-block counts (the causal mirrored pairs), non-causal, eps > 0,
both head mappings (BH a multiple of 8 or not), decay and rotary Q.  The
benchmark workload's shape at these widths (B8 H16 T4096, causal, rotary
inputs) runs in the benchmark's launch configuration and is checked on
sampled rows, and its output is bitwise the same over repeated calls.
"""
import dataclasses

import numpy as np
import pytest

from complex_valued_attention_amd import inputs as gen
from complex_valued_attention_amd.check import TOL, from_device, rowwise_rel_err, sample_rows, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

WIDTHS = [128, 32]


def _cattn():
    from complex_valued_attention_amd import cattn
    cattn.lib()   # fail loudly if the HIP library is missing
    return cattn


def say(*a):
    print(*a, flush=True)


CASES = [
    # (causal, B, H, T, eps)
    (True, 1, 1, 1, 0.0),
    (True, 1, 2, 15, 0.0),
    (True, 1, 2, 16, 0.0),
    (True, 1, 2, 17, 0.0),
    (True, 1, 2, 33, 0.0),
    (True, 1, 2, 127, 0.0),
    (True, 1, 2, 128, 0.0),
    (True, 1, 2, 129, 0.0),
    (True, 1, 2, 300, 0.0),
    (True, 1, 2, 385, 0.0),
    (True, 1, 1, 513, 0.0),
    (True, 2, 4, 260, 0.0),     # BH = 8: the XCD head mapping
    (True, 1, 3, 200, 0.3),
    (False, 1, 1, 1, 0.0),
    (False, 1, 2, 31, 0.0),
    (False, 1, 2, 100, 0.0),
    (False, 1, 2, 257, 0.0),
    (False, 2, 4, 130, 0.1),
]


@pytest.mark.parametrize("D", WIDTHS)
@pytest.mark.parametrize("causal,B,H,T,eps", CASES)
def test_born_bf16_q16_small(D, causal, B, H, T, eps):
    import oracle
    c = _cattn()
    w = gen.Workload("q16", "born", causal, B, H, T, D, "bf16", seed=61, qk_unit=True, rotary=True)
    say("case q16", w, eps)
    inp = gen.make_inputs(w)
    q, k, v = to_device(inp)
    den = torch.full((B * H * T,), float("nan"), dtype=torch.float32, device="cuda")
    o = c.born_fwd(q, k, v, causal=causal, eps=eps, row_den=den)
    torch.cuda.synchronize()
    ref, rden = oracle.born_attention(inp.q64, inp.k64, inp.v64, causal=causal, eps=eps, return_den=True)
    err = rowwise_rel_err(from_device(o), ref)
    say(f"q16 d{D} causal={causal} B{B} H{H} T{T} eps={eps}: rowwise rel err {err:.3e}")
    assert err <= TOL["bf16"]
    gd = den.cpu().numpy().reshape(B, H, T).astype(np.float64)
    np.testing.assert_allclose(gd, rden, rtol=2e-2)


@pytest.mark.parametrize("T,gammas", [(300, (0.9, 0.995)), (129, (0.5, 1.0))])
@pytest.mark.parametrize("D", WIDTHS)
def test_born_bf16_q16_decay(D, T, gammas):
    import oracle
    c = _cattn()
    w = gen.Workload("q16d", "born", True, 1, 2, T, D, "bf16", seed=62, qk_unit=True, rotary=True)
    say("case q16 decay", w, gammas)
    inp = gen.make_inputs(w)
    q, k, v = to_device(inp)
    o = c.born_fwd(q, k, v, causal=True, decay=list(gammas))
    torch.cuda.synchronize()
    g32 = np.asarray(gammas, dtype=np.float32).astype(np.float64)
    ref = oracle.born_attention(inp.q64, inp.k64, inp.v64, causal=True, decay=g32)
    err = rowwise_rel_err(from_device(o), ref)
    say(f"q16 decay d{D} T{T}: rowwise rel err {err:.3e}")
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("T,pos0", [(300, 0), (77, 123_457)])
@pytest.mark.parametrize("D", WIDTHS)
def test_born_bf16_q16_rotary_q(D, T, pos0):
    # rotary Q in the kernel against the rotary pass over Q followed by the plain kernel
    c = _cattn()
    w = gen.Workload("q16r", "born", True, 1, 2, T, D, "bf16", seed=63, qk_unit=True)
    say("case q16 rotary", w, pos0)
    inp = gen.make_inputs(w)
    q, k, v = to_device(inp)
    o_in = c.born_fwd(q, k, v, causal=True, rotary_base=10000.0, rotary_pos0=pos0)
    qr = c.rotary(q, base=10000.0, pos0=pos0)
    o_pass = c.born_fwd(qr, k, v, causal=True)
    torch.cuda.synchronize()
    a, b = from_device(o_in), from_device(o_pass)
    err = rowwise_rel_err(a, b)
    say(f"q16 rotary d{D} T{T} pos0 {pos0}: in-kernel vs pass {err:.3e}")
    assert err <= 1e-2


@pytest.mark.parametrize("D", WIDTHS)
def test_born_bf16_q16_full_size_sampled_and_deterministic(D):
    import oracle
    c = _cattn()
    w = dataclasses.replace(gen.WORKLOADS["born_causal_bf16_b8h16t4096d64_rotary"], d_h=D)
    say("case q16 full", w)
    inp = gen.make_inputs(w)
    q, k, v = to_device(inp)
    o1 = c.born_fwd(q, k, v, causal=True)
    o2 = c.born_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    got = from_device(o1)
    assert np.isfinite(got).all()
    for a, b in zip(o1, o2):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    rows = sample_rows(w.B, w.H, w.T, 96, seed=w.seed, tile=128)
    ref = oracle.born_attention_rows(inp.q64, inp.k64, inp.v64, rows, causal=True)
    err = rowwise_rel_err(got[rows[:, 0], rows[:, 1], rows[:, 2]], ref)
    say(f"q16 d{D} full size, {len(rows)} sampled rows: rowwise rel err {err:.3e}")
    assert err <= TOL["bf16"]
