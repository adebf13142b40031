"""GPU parity of the forward calls on strided operands.

The pages' BornAttention layer ("Show HN: CNET", BornAttention) takes Q, K
and V as one concatenated input.  Here they are views of one fused projection
output laid out [B, T, 3, H, d_h], and O is a view of a [B, T, H, d_h]
buffer, so the calls see token strides of 3·H·d_h and H·d_h and head strides
of d_h.  Every case is checked against the fp64 oracle.  Where every stride is
a multiple of 16 bytes the same matrix-core kernel runs as for dense tensors,
so the output must also equal the dense call's bit for bit; other strides take
the element-wise kernel.
"""
import dataclasses

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


def say(*a):
    print(*a, flush=True)


def _fuse(xs, pad=0):
    """Views of one [B, T, 3, H, d_h + pad] buffer holding the three [B, H, T, d_h]
    tensors xs, each view [B, H, T, d_h] (the last `pad` components unused)."""
    B, H, T, d = xs[0].shape
    f = torch.full((B, T, 3, H, d + pad), float("nan"), dtype=xs[0].dtype, device=xs[0].device)
    if f.is_complex():
        f = torch.full((B, T, 3, H, d + pad), complex(float("nan"), 0.0), dtype=xs[0].dtype, device=xs[0].device)
    views = []
    for i, x in enumerate(xs):
        v = f[:, :, i, :, :d].permute(0, 2, 1, 3)
        v.copy_(x)
        views.append(v)
    return views


def fused_operands(q, k, v, pad=0):
    """q, k, v (complex64 tensors or bf16 plane pairs) as views of fused buffers."""
    if isinstance(q, tuple):
        re = _fuse([q[0], k[0], v[0]], pad)
        im = _fuse([q[1], k[1], v[1]], pad)
        return tuple((re[i], im[i]) for i in range(3))
    return tuple(_fuse([q, k, v], pad))


def strided_out(like, pad=0):
    """An output view [B, H, T, d_h] of a NaN-filled [B, T, H, d_h + pad] buffer."""
    def one(x):
        B, H, T, d = x.shape
        fill = complex(float("nan"), 0.0) if x.is_complex() else float("nan")
        buf = torch.full((B, T, H, d + pad), fill, dtype=x.dtype, device=x.device)
        return buf[..., :d].permute(0, 2, 1, 3)
    if isinstance(like, tuple):
        return (one(like[0]), one(like[1]))
    return one(like)


def call(c, w, q, k, v, out=None, gate=None):
    if w.op == "born":
        o = c.born_fwd(q, k, v, causal=w.causal, out=out)
    elif gate is None:
        o = c.pct_fwd(q, k, v, causal=w.causal, out=out)
    else:
        o = c.pct_gate_fwd(q, k, v, gate=gate, causal=w.causal, out=out)
    torch.cuda.synchronize()
    return o


def oracle_out(w, inp, rows=None, gate=None):
    import oracle
    if rows is not None:
        fn = oracle.born_attention_rows if w.op == "born" else oracle.pct_attention_rows
        return fn(inp.q64, inp.k64, inp.v64, rows, causal=w.causal)
    if w.op == "born":
        return oracle.born_attention(inp.q64, inp.k64, inp.v64, causal=w.causal)
    if gate == "softmax":
        return oracle.pct_softmax_attention(inp.q64, inp.k64, inp.v64, causal=w.causal)
    return oracle.pct_attention(inp.q64, inp.k64, inp.v64, causal=w.causal)


def same_bits(a, b):
    if isinstance(a, tuple):
        return all(torch.equal(x.contiguous().view(torch.int16), y.contiguous().view(torch.int16))
                   for x, y in zip(a, b))
    return torch.equal(torch.view_as_real(a.contiguous()).view(torch.int32),
                       torch.view_as_real(b.contiguous()).view(torch.int32))


# (workload, B, H, T, d_h, layout override, gate) -- small sizes, every row checked
SMALL = [
    ("born_causal_c64_b4h8t1024d64_rotary", 1, 3, 300, 64, None, None),    # complex64 matrix-core kernel
    ("born_causal_bf16_b8h16t4096d64_rotary", 1, 3, 300, 64, None, None),  # the bf16 width-64 kernel
    ("born_causal_bf16_b8h16t4096d64_rotary", 2, 2, 1000, 64, None, None),
    ("pct_full_c64_b8h8t2048d64", 1, 2, 300, 64, None, None),
    ("pct_causal_c64_b1h8t16384d64", 1, 2, 300, 32, "bf16", None),         # PCT on bf16 planes
    ("pct_full_c64_b8h8t2048d64", 1, 2, 200, 16, None, "softmax"),
    ("born_causal_bf16_b8h16t4096d64_rotary", 1, 2, 257, 16, None, None),  # bf16 widths 16/32/128
    ("born_causal_bf16_b8h16t4096d64_rotary", 1, 2, 257, 32, None, None),
    ("born_causal_bf16_b8h16t4096d64_rotary", 1, 1, 300, 128, None, None),
    ("born_causal_c64_b1h1t128d16", 2, 3, 100, 16, None, None),
]


@pytest.mark.parametrize("name,B,H,T,d,layout,gate", SMALL,
                         ids=[f"{s[0]}-B{s[1]}H{s[2]}T{s[3]}d{s[4]}-{s[5] or 'same'}-{s[6] or 'plain'}"
                              for s in SMALL])
def test_fused_views_small(name, B, H, T, d, layout, gate):
    c = _cattn()
    w = dataclasses.replace(gen.WORKLOADS[name], B=B, H=H, T=T, d_h=d, **({"layout": layout} if layout else {}))
    say("case strided", w, gate)
    inp = gen.make_inputs(w)
    q, k, v = to_device(inp)
    dense = call(c, w, q, k, v, gate=gate)
    fq, fk, fv = fused_operands(q, k, v)
    out = strided_out(dense)
    got = call(c, w, fq, fk, fv, out=out, gate=gate)
    ref = oracle_out(w, inp, gate=gate)
    err = rowwise_rel_err(from_device(tuple(x.contiguous() for x in got) if isinstance(got, tuple)
                                      else got.contiguous()), ref)
    say(f"strided {w.op} {w.layout} B{B} H{H} T{T} d{d}: rowwise rel err {err:.3e}")
    assert err <= TOL[w.layout]
    # 16-byte strides: the dense call's kernel, so the same bits
    assert same_bits(got, dense)


# element strides that are not a multiple of 16 bytes: the element-wise kernel
ODD = [
    ("born", "c64", True, 1, 2, 130, 64, 1),
    ("born", "bf16", True, 1, 2, 130, 64, 3),
    ("pct", "c64", False, 2, 1, 77, 32, 1),
    ("pct", "bf16", True, 1, 2, 90, 16, 5),
]


@pytest.mark.parametrize("op,layout,causal,B,H,T,d,pad", ODD)
def test_fused_views_unaligned_strides(op, layout, causal, B, H, T, d, pad):
    c = _cattn()
    w = gen.Workload("strided", op, causal, B, H, T, d, layout, seed=11)
    say("case odd strides", w, pad)
    inp = gen.make_inputs(w)
    q, k, v = to_device(inp)
    fq, fk, fv = fused_operands(q, k, v, pad=pad)
    out = strided_out(q, pad=pad)
    got = call(c, w, fq, fk, fv, out=out)
    ref = oracle_out(w, inp)
    err = rowwise_rel_err(from_device(tuple(x.contiguous() for x in got) if isinstance(got, tuple)
                                      else got.contiguous()), ref)
    say(f"odd strides {op} {layout} pad {pad}: rowwise rel err {err:.3e}")
    assert err <= TOL[layout]


def test_fused_views_mixed_operands():
    # each operand with strides of its own: Q fused, K a slice of a wider buffer, V dense, O fused
    c = _cattn()
    w = dataclasses.replace(gen.WORKLOADS["born_causal_bf16_b8h16t4096d64_rotary"], B=2, H=2, T=333)
    inp = gen.make_inputs(w)
    q, k, v = to_device(inp)
    fq, _, _ = fused_operands(q, k, v)
    wide = tuple(torch.zeros(w.B, w.H, w.T, 2 * w.d_h, dtype=torch.bfloat16, device="cuda") for _ in range(2))
    for p in range(2):
        wide[p][..., w.d_h:].copy_(k[p])
    kk = tuple(x[..., w.d_h:] for x in wide)
    out = strided_out(q)
    got = c.born_fwd(fq, kk, v, causal=True, out=out)
    dense = c.born_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    err = rowwise_rel_err(from_device(tuple(x.contiguous() for x in got)), oracle_out(w, inp))
    say(f"mixed operand strides: rowwise rel err {err:.3e}")
    assert err <= TOL["bf16"]
    assert same_bits(got, dense)


@pytest.mark.parametrize("name", ["born_causal_c64_b4h8t1024d64_rotary", "born_causal_bf16_b8h16t4096d64_rotary"])
def test_fused_views_full_size(name):
    # the workloads at full size on views of one fused buffer: sampled rows
    # against the oracle, and every row bit for bit against the dense call
    c = _cattn()
    w = gen.WORKLOADS[name]
    say("case strided full", w)
    inp = gen.make_inputs(w)
    q, k, v = to_device(inp)
    dense = call(c, w, q, k, v)
    fq, fk, fv = fused_operands(q, k, v)
    del q, k, v
    out = strided_out(dense)
    got = call(c, w, fq, fk, fv, out=out)
    assert same_bits(got, dense)
    g = from_device(tuple(x.contiguous() for x in got) if isinstance(got, tuple) else got.contiguous())
    rows = sample_rows(w.B, w.H, w.T, 64, seed=w.seed)
    ref = oracle_out(w, inp, rows=rows)
    err = rowwise_rel_err(g[rows[:, 0], rows[:, 1], rows[:, 2]], ref)
    say(f"{name} on fused views: {len(rows)} sampled rows, rowwise rel err {err:.3e}")
    assert err <= TOL[w.layout]
