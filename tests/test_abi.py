"""The C-ABI library: it loads, exports every function include/cattn.h declares,
and rejects bad arguments before any HIP call (CPU only, no kernel runs)."""
import ctypes
import os
import re

import pytest

from complex_valued_attention_amd import cattn

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "cattn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(cattn.LIB_PATH), reason="libcattn.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cattn_\w+)\s*\(", text)))


def test_header_declares_entry_points():
    assert declared_functions() == ["cattn_abi_version", "cattn_born_bwd", "cattn_born_fwd", "cattn_born_merge",
                                    "cattn_born_state", "cattn_born_step", "cattn_pct_bwd", "cattn_pct_fwd",
                                    "cattn_pct_gate_fwd", "cattn_rotary", "cattn_status_str"]


def test_library_exports_every_declared_symbol():
    L = cattn.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert L.cattn_abi_version() == 8


def test_status_strings():
    L = cattn.lib()
    for s in range(0, 9):
        assert L.cattn_status_str(s)
    assert L.cattn_status_str(12345) == b"unknown status"


# fake, aligned, never dereferenced addresses: each call below must fail validation first
P = [0x100000 * (i + 1) for i in range(8)]


def strides(q=(0, 0, 0), k=(0, 0, 0), v=(0, 0, 0), o=(0, 0, 0)):
    return ctypes.byref(cattn.Strides(cattn.Stride(*q), cattn.Stride(*k), cattn.Stride(*v), cattn.Stride(*o)))


def born(layout=0, ptrs=None, B=1, H=1, T=8, d=4, causal=1, eps=0.0, row_den=None, st=None, opts=None):
    q = ptrs if ptrs is not None else ([P[0], None, P[1], None, P[2], None, P[3], None] if layout == 0 else P)
    return cattn.lib().cattn_born_fwd(layout, *q, B, H, T, d, st, causal, eps, row_den, opts, None)


def pct(layout=0, ptrs=None, B=1, H=1, T=8, d=4, causal=0, bias=0.0, st=None):
    q = ptrs if ptrs is not None else ([P[0], None, P[1], None, P[2], None, P[3], None] if layout == 0 else P)
    return cattn.lib().cattn_pct_fwd(layout, *q, B, H, T, d, st, causal, bias, None)


def test_bad_layout():
    assert born(layout=7) == 3
    assert pct(layout=-1) == 3


def test_bad_sizes():
    assert born(B=-1) == 2
    assert born(T=-5) == 2
    assert born(d=0) == 6
    assert born(d=129) == 6
    assert pct(d=1000) == 6
    assert born(T=2 ** 40) == 2
    assert born(T=2 ** 30 + 1) == 2      # past CATTN_MAX_T
    assert born(B=2 ** 20, H=2 ** 20, T=2 ** 20) == 2


def test_empty_problem_is_ok_and_launches_nothing():
    # B, H or T equal to 0: OK, and pointers may even be NULL
    assert born(ptrs=[None] * 8, B=0) == 0
    assert pct(ptrs=[None] * 8, T=0) == 0
    assert born(ptrs=[None] * 8, H=0, layout=1) == 0


def test_null_pointers():
    assert born(ptrs=[None, None, P[1], None, P[2], None, P[3], None]) == 1
    assert born(ptrs=[P[0], None, P[1], None, P[2], None, None, None]) == 1
    # C64 must not carry imaginary-plane pointers
    assert born(ptrs=[P[0], P[4], P[1], None, P[2], None, P[3], None]) == 1
    # bf16 needs both planes
    assert born(layout=1, ptrs=[P[0], None, P[1], P[5], P[2], P[6], P[3], P[7]]) == 1


def test_alignment():
    # the forward calls need element alignment: 8 bytes (complex64), 2 (bf16), 4 (row_den)
    assert born(ptrs=[P[0] + 4, None, P[1], None, P[2], None, P[3], None]) == 4
    assert pct(layout=1, ptrs=[P[0], P[1], P[2], P[3], P[4], P[5], P[6], P[7] + 1]) == 4
    assert born(row_den=P[7] + 2) == 4


def test_aliasing():
    # O overlapping Q
    assert born(ptrs=[P[0], None, P[1], None, P[2], None, P[0] + 16, None]) == 5
    # bf16: O real and imaginary planes overlapping each other
    assert born(layout=1, ptrs=[P[0], P[1], P[2], P[3], P[4], P[5], P[6], P[6] + 16]) == 5
    # row_den overlapping O
    assert born(row_den=P[3]) == 5


def test_bad_scalars():
    assert born(eps=-1.0) == 8
    assert born(eps=float("nan")) == 8
    assert born(eps=float("inf")) == 8
    assert pct(bias=float("nan")) == 8
    assert pct(bias=float("-inf")) == 8


def test_strides_validation():
    # negative strides
    assert born(st=strides(q=(0, 0, -4))) == 2
    assert pct(st=strides(o=(-1, 0, 0)), B=2) == 2
    # an extent past int64
    assert born(st=strides(k=(0, 0, 2 ** 62)), T=8) == 2
    # rows of O sharing memory: token stride below the row width, or heads on top of each other
    assert born(st=strides(o=(0, 0, 2)), d=4) == 5
    assert born(st=strides(o=(0, 8, 4)), H=2, T=4, d=4) == 5
    # O's span reaching into an input: Q dense at P0 (8 rows of 4 = 256 B), O from P0 + 256 - 16
    assert born(ptrs=[P[0], None, P[1], None, P[2], None, P[0] + 240, None]) == 5
    # strides stretch spans: K at P1 with token stride 2^20 elements reaches far past O at P3
    assert born(st=strides(k=(0, 0, 2 ** 20))) == 5
    # row_den inside a strided input's span
    assert born(st=strides(v=(0, 0, 2 ** 20)), row_den=P[5]) == 5
    # with a stride, the other checks still come first: NULL, alignment
    assert born(st=strides(q=(0, 0, 8)), ptrs=[None, None, P[1], None, P[2], None, P[3], None]) == 1
    assert born(st=strides(q=(0, 0, 8)), ptrs=[P[0] + 4, None, P[1], None, P[2], None, P[3], None]) == 4


def test_python_binding_rejects_bad_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 1, 4, 4, dtype=torch.complex64)
    with pytest.raises(ValueError):
        cattn.born_fwd(x, x, x)            # host tensors are refused before any call
    with pytest.raises(TypeError):
        cattn.born_fwd(x.real, x.real, x.real)
    # per-row float32 buffers (row_den, db_rows): dtype, device, size and layout are checked
    dev = torch.device("cuda", 0)
    with pytest.raises(ValueError, match="must be on"):
        cattn._rows_f32(torch.zeros(8), 8, dev, "row_den")                     # a host tensor
    with pytest.raises(TypeError, match="float32"):
        cattn._rows_f32(torch.zeros(8, dtype=torch.bfloat16), 8, dev, "row_den")
    with pytest.raises(TypeError, match="float32"):
        cattn._rows_f32(torch.zeros(8, dtype=torch.float64), 8, dev, "row_den")
    with pytest.raises(ValueError, match="8 elements"):
        cattn._rows_f32(torch.zeros(7), 8, torch.device("cpu"), "row_den")
    with pytest.raises(ValueError, match="8 elements"):
        cattn._rows_f32(torch.zeros(16)[::2], 8, torch.device("cpu"), "row_den")
    assert cattn._rows_f32(torch.zeros(8), 8, torch.device("cpu"), "row_den") is not None
    # the carried state: dtype and device
    with pytest.raises(ValueError, match="must be on"):
        cattn._state_ptr(torch.zeros(1, 1, 3, 1, 1), 1, 1, 1, dev)
    with pytest.raises(TypeError):
        cattn._state_ptr(torch.zeros(1, 1, 3, 1, 1, dtype=torch.float64), 1, 1, 1, torch.device("cpu"))
    # strides: a broadcast view is refused, a slice of a fused buffer passes through as it is
    with pytest.raises(ValueError, match="broadcast"):
        cattn._stride3(torch.zeros(1, 1, 4, 4).expand(2, 1, 4, 4), "k")
    fused = torch.zeros(2, 5, 3, 4, 8)           # [B, T, 3, H, d]
    qv = fused[:, :, 0].permute(0, 2, 1, 3)      # [B, H, T, d] view
    st = cattn._stride3(qv, "q")
    assert (st.b, st.h, st.t) == (5 * 3 * 4 * 8, 8, 3 * 4 * 8)


# ---- backward entry points -------------------------------------------------
Q = [0x100000 * (i + 20) for i in range(16)]


def born_b(layout=0, ins=None, outs=None, row_den=Q[15], B=1, H=1, T=8, d=4, causal=1, decay=None):
    if ins is None:   # q, k, v, o, g as (re, im) pairs
        ins = [(Q[i], None) for i in range(5)] if layout == 0 else [(Q[i], Q[i + 5]) for i in range(5)]
    if outs is None:  # dq, dk, dv
        outs = [(Q[10 + i], None if layout == 0 else 0x100000 * (41 + i)) for i in range(3)]
    flat_in = [x for pair in ins for x in pair]
    flat_out = [x for pair in outs for x in pair]
    return cattn.lib().cattn_born_bwd(layout, *flat_in, row_den, *flat_out, B, H, T, d, causal, decay, None)


def pct_b(layout=0, ins=None, outs=None, db_rows=None, B=1, H=1, T=8, d=4, causal=0, bias=0.0):
    if ins is None:   # q, k, v, g
        ins = [(Q[i], None) for i in range(4)] if layout == 0 else [(Q[i], Q[i + 5]) for i in range(4)]
    if outs is None:
        outs = [(Q[10 + i], None) for i in range(3)]
    flat_in = [x for pair in ins for x in pair]
    flat_out = [x for pair in outs for x in pair]
    return cattn.lib().cattn_pct_bwd(layout, *flat_in, *flat_out, B, H, T, d, causal, bias, db_rows, None)


def test_bwd_argument_errors():
    assert born_b(layout=5) == 3
    assert pct_b(d=0) == 6
    assert born_b(T=-1) == 2
    assert pct_b(bias=float("nan")) == 8
    # Born needs O, G and row_den
    assert born_b(row_den=None) == 1
    ins = [(Q[i], None) for i in range(5)]
    ins[3] = (None, None)
    assert born_b(ins=ins) == 1
    # PCT needs G
    ins = [(Q[i], None) for i in range(4)]
    ins[3] = (None, None)
    assert pct_b(ins=ins) == 1
    # complex64 carries no imaginary planes
    outs = [(Q[10], Q[13]), (Q[11], None), (Q[12], None)]
    assert pct_b(outs=outs) == 1
    # alignment of an output and of db_rows
    outs = [(Q[10] + 8, None), (Q[11], None), (Q[12], None)]
    assert born_b(outs=outs) == 4
    assert pct_b(db_rows=Q[14] + 4) == 4


def test_bwd_aliasing():
    # dq over k
    outs = [(Q[1], None), (Q[11], None), (Q[12], None)]
    assert born_b(outs=outs) == 5
    # dk over dv
    outs = [(Q[10], None), (Q[11], None), (Q[11] + 16, None)]
    assert pct_b(outs=outs) == 5
    # db_rows over an output
    assert pct_b(db_rows=Q[12]) == 5
    # an output over row_den
    outs = [(Q[10], None), (Q[15], None), (Q[12], None)]
    assert born_b(outs=outs) == 5


def test_bwd_empty_problem_is_ok():
    assert born_b(ins=[(None, None)] * 5, outs=[(None, None)] * 3, row_den=None, T=0) == 0
    assert pct_b(ins=[(None, None)] * 4, outs=[(None, None)] * 3, B=0) == 0


def gate_fwd(gate, a=0.0, b=0.0, layout=0, T=8, misalign=0):
    # every call must fail validation: a misaligned O stops the ones whose gate arguments pass
    q = [P[0], None, P[1], None, P[2], None, P[3] + misalign, None] if layout == 0 else P
    return cattn.lib().cattn_pct_gate_fwd(layout, *q, 1, 1, T, 4, None, 1, gate, a, b, None)


def test_gate_arguments():
    assert gate_fwd(3) == 8                    # unknown gate
    assert gate_fwd(-1) == 8
    assert gate_fwd(0, a=float("nan")) == 8    # sigmoid bias
    assert gate_fwd(2, a=float("inf")) == 8    # screening r
    assert gate_fwd(2, b=float("nan")) == 8    # screening t
    assert gate_fwd(1, a=float("nan"), misalign=4) == 4   # the softmax gate ignores a and b
    assert gate_fwd(1, T=0) == 0


def rot(layout=0, ptrs=None, B=1, H=1, T=8, d=4, pos0=0, base=10000.0):
    xs = ptrs if ptrs is not None else ([P[0], None, P[1], None] if layout == 0 else [P[0], P[1], P[2], P[3]])
    return cattn.lib().cattn_rotary(layout, *xs, B, H, T, d, pos0, base, None)


def test_rotary_argument_errors():
    # every call fails validation (or is empty): none reaches a launch
    assert rot(layout=9) == 3
    assert rot(base=0.0) == 8
    assert rot(base=float("nan")) == 8
    assert rot(pos0=-1) == 8
    assert rot(pos0=2 ** 41) == 8
    assert rot(d=0) == 6
    assert rot(T=-2) == 2
    assert rot(T=0) == 0
    assert rot(ptrs=[P[0], P[4], P[1], None]) == 1          # complex64 takes no imaginary plane
    assert rot(layout=1, ptrs=[P[0], None, P[2], P[3]]) == 1
    assert rot(ptrs=[P[0], None, P[1] + 8, None]) == 4
    assert rot(ptrs=[P[0], None, P[0] + 16, None]) == 5     # partial overlap of input and output
    assert rot(layout=1, ptrs=[P[0], P[1], P[1], P[2]]) == 5   # output real plane over the input imaginary plane


S = [0x1000000 * (i + 2) for i in range(10)]   # far apart: state buffers are large


def test_linear_argument_errors():
    L = cattn.lib()
    # state build: d_h above 64 is unsupported for the carried state
    assert L.cattn_born_state(0, S[0], None, S[1], None, 1, 1, 8, 65, S[2], 0, None, None) == 6
    assert L.cattn_born_state(0, S[0], None, S[1], None, 1, 1, 8, 4, None, 0, None, None) == 1
    assert L.cattn_born_state(0, S[0], None, S[1], None, 1, 1, 8, 4, S[2] + 8, 0, None, None) == 4
    assert L.cattn_born_state(0, S[0], None, S[1], None, 1, 1, 8, 4, S[0] + 16, 0, None, None) == 5   # state over k
    assert L.cattn_born_state(0, S[0], None, S[1], None, 1, 1, 0, 4, None, 1, None, None) == 0        # empty
    assert L.cattn_born_state(0, None, None, None, None, 1, 1, 0, 4, None, 0, None, None) == 1        # zeroing needs S
    assert L.cattn_born_state(0, None, None, None, None, 0, 1, 0, 4, None, 0, None, None) == 0        # no heads
    # merge: the written output and row_den must not overlap the state
    assert L.cattn_born_merge(0, S[0], None, S[1], S[1], None, S[4], 1, 1, 8, 4, None, None) == 5
    assert L.cattn_born_merge(0, S[0], None, S[1], S[3], None, None, 1, 1, 8, 4, None, None) == 1
    # step: eps checked first; o over q
    assert L.cattn_born_step(0, S[0], None, S[1], None, S[2], None, S[3], None, S[4], S[6], 1, 1, 4,
                             -1.0, None, None) == 8
    assert L.cattn_born_step(0, S[0], None, S[1], None, S[2], None, S[0], None, S[4], S[6], 1, 1, 4,
                             0.0, None, None) == 5
    assert L.cattn_born_step(1, S[0], None, S[1], S[7], S[2], S[8], S[3], S[9], S[4], S[6], 1, 1, 4,
                             0.0, None, None) == 1   # bf16 needs both planes of q


def _floats(*v):
    return (ctypes.c_float * len(v))(*v)


def _opts(decay=None, base=0.0, pos0=0):
    d = None if decay is None else ctypes.cast(decay, ctypes.POINTER(ctypes.c_float))
    return ctypes.byref(cattn.BornOpts(d, base, pos0))


def test_born_options_validation():
    # every case is valid but for its options, so each must stop there, before any launch
    H = 3
    ok = _floats(0.5, 1.0, 0.99)
    for bad in ((0.5, 0.0, 0.9), (0.5, -0.1, 0.9), (1.0, 1.5, 0.9), (float("nan"), 0.5, 0.5),
                (float("inf"), 0.5, 0.5)):
        assert born(H=H, opts=_opts(_floats(*bad))) == 8, bad
    assert born(H=H, causal=0, opts=_opts(ok)) == 8                 # decay needs causal attention
    assert born(H=257, opts=_opts(_floats(*([0.5] * 257)))) == 6      # more heads than a table holds
    assert born(H=H, opts=_opts(base=-1.0)) == 8
    assert born(H=H, opts=_opts(base=float("nan"))) == 8
    assert born(H=H, opts=_opts(base=float("inf"))) == 8
    assert born(H=H, opts=_opts(base=10000.0, pos0=-1)) == 8
    assert born(H=H, opts=_opts(base=10000.0, pos0=(1 << 40) + 1)) == 8
    assert born(B=0, H=H, opts=_opts(_floats(0.5, 2.0, 0.5))) == 8    # options are checked on empty calls too
    assert born(B=0, H=H, opts=_opts(ok, base=10000.0)) == 0        # empty and valid: nothing to do
    # the argument checks of the call itself come first
    assert born(H=H, d=0, opts=_opts(_floats(0.5, 2.0, 0.5))) == 6


def test_decay_validation_backward_and_state():
    L = cattn.lib()
    bad = _floats(0.5, 0.0)
    assert born_b(H=2, decay=bad) == 8
    assert born_b(H=2, causal=0, decay=_floats(0.5, 0.5)) == 8
    assert born_b(H=300, decay=_floats(*([0.5] * 300))) == 6
    # carried state: a bad table is refused before anything else is looked at
    assert L.cattn_born_state(0, S[0], None, S[1], None, 1, 2, 8, 4, S[2], 0, bad, None) == 8
    assert L.cattn_born_merge(0, S[0], None, S[1], S[3], None, S[4], 1, 2, 8, 4, bad, None) == 8
    assert L.cattn_born_step(0, S[0], None, S[1], None, S[2], None, S[3], None, S[4], S[6], 1, 2, 4, 0.0, bad,
                             None) == 8
    assert L.cattn_born_state(0, S[0], None, S[1], None, 1, 257, 8, 4, S[2], 0, _floats(*([0.5] * 257)),
                              None) == 6


def test_binding_decay_table():
    arr = cattn._decay([0.5, 0.25], 2)
    assert list(arr) == [0.5, 0.25]
    assert list(cattn._decay(0.75, 3)) == [0.75, 0.75, 0.75]
    assert cattn._decay(None, 4) is None
    with pytest.raises(ValueError):
        cattn._decay([0.5], 2)
