"""GPU parity of the rotary phase embedding ("Show HN: CNET", RotaryEmbed)
against the fp64 oracle, through the C ABI, on seeded inputs: both layouts,
vector and scalar channel paths, long positions, in place and not."""
import numpy as np
import pytest

from complex_valued_attention_amd import inputs as gen
from complex_valued_attention_amd.check import TOL, from_device, rowwise_rel_err, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

CASES = [
    # (layout, B, H, T, d, pos0, base)
    ("c64", 1, 2, 300, 64, 0, 10000.0),
    ("c64", 2, 1, 77, 16, 5, 10000.0),
    ("c64", 1, 1, 100, 3, 0, 10000.0),        # odd width: scalar path
    ("c64", 1, 1, 16384, 64, 0, 10000.0),     # long positions
    ("c64", 1, 1, 64, 128, 1_000_000, 500.0),  # large offset, other base
    ("bf16", 1, 2, 300, 64, 0, 10000.0),
    ("bf16", 1, 1, 100, 17, 3, 10000.0),      # scalar path
    ("bf16", 1, 1, 4096, 128, 123_457, 10000.0),
    ("c64", 1, 1, 1, 64, 42, 10000.0),
]


def say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("layout,B,H,T,d,pos0,base", CASES)
@pytest.mark.parametrize("inplace", [False, True])
def test_rotary_parity(layout, B, H, T, d, pos0, base, inplace):
    import oracle
    from complex_valued_attention_amd import cattn
    w = gen.Workload("rot", "born", True, B, H, T, d, layout, seed=61)
    inp = gen.make_inputs(w)
    x = to_device(inp)[0]
    y = cattn.rotary(x, pos0=pos0, base=base, out=x if inplace else None)
    torch.cuda.synchronize()
    got = from_device(y)
    ref = oracle.rotary(inp.q64, pos0=pos0, base=base)
    err = rowwise_rel_err(got, ref)
    say(f"rotary {layout} B{B} H{H} T{T} d{d} pos0={pos0} base={base} inplace={inplace}: {err:.3e}")
    assert err <= TOL[layout]


def test_rotary_then_born_equals_born_of_rotated_inputs():
    # the device pass reproduces the host recipe of the rotary workloads
    from complex_valued_attention_amd import cattn
    import oracle
    w = gen.Workload("rotb", "born", True, 1, 2, 520, 64, "c64", seed=62, qk_unit=True)
    inp = gen.make_inputs(w)
    q, k, v = to_device(inp)
    o = cattn.born_fwd(cattn.rotary(q), cattn.rotary(k), v, causal=True)
    torch.cuda.synchronize()
    ref = oracle.born_attention(oracle.rotary(inp.q64), oracle.rotary(inp.k64), inp.v64, causal=True)
    assert rowwise_rel_err(from_device(o), ref) <= TOL["c64"]
