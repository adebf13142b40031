"""GPU parity of Born attention with a carried density state ("Show HN: CNET",
BornAttention's linear and step modes) against the fp64 oracle, through the C
ABI: the state build (overwrite and accumulate), a sequence split over two
calls with the first part carried as a state, token-by-token decoding, and the
zero-denominator case.  The device state is the packed real form of the
oracle's (Z, M) (fp32 in both layouts); it is compared with the oracle's state
after packing (``oracle.pack_state``)."""
import numpy as np
import pytest

from complex_valued_attention_amd import inputs as gen
from complex_valued_attention_amd.check import GRAD_FLOOR, TOL, from_device, rowwise_rel_err, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

def state_tol(layout, d):
    """fp32 sums of the rounded inputs: 1e-4.  bf16 planes at width 64 run on
    the matrix cores, which round every lifted feature Re/Im(k_a conj k_b) to
    bf16 (2^-9 relative per term) before the fp32 sum: the output bar."""
    return TOL["bf16"] if (layout == "bf16" and d == 64) else 1e-4
# Row denominators: the bf16 forward sums the bf16-rounded weights it applies
# to V (each within 2^-9 relative, all positive, so the sum is too).
DEN_TOL = {"c64": 1e-5, "bf16": 2.0 ** -8}


def say(*a):
    print(*a, flush=True)


def _slice(x, t0, t1):
    # a fresh allocation: a slice of a one-head tensor is a contiguous view at
    # an offset that need not meet the 16-byte alignment of operand bases
    if isinstance(x, tuple):
        return tuple(p[:, :, t0:t1].clone(memory_format=torch.contiguous_format) for p in x)
    return x[:, :, t0:t1].clone(memory_format=torch.contiguous_format)


def _oracle_state(inp, B, H, t0, t1):
    """The oracle's packed state [B, H, 2d + 1, d, d] of tokens t0 .. t1 - 1."""
    import oracle
    d = inp.k64.shape[-1]
    S = np.zeros((B, H, 2 * d + 1, d, d))
    for b in range(B):
        for h in range(H):
            S[b, h] = oracle.pack_state(*oracle.born_state(inp.k64[b, h, t0:t1], inp.v64[b, h, t0:t1]))
    return S


def _state_err(Sg, S):
    """Row-wise error of each packed matrix (rows of d features), scaled per tensor."""
    return rowwise_rel_err(Sg.cpu().numpy().astype(np.float64), S, floor=GRAD_FLOOR)


STATE_CASES = [
    # (layout, B, H, T, d)
    ("c64", 1, 2, 200, 16),
    ("c64", 1, 1, 130, 17),
    ("c64", 2, 1, 64, 33),
    ("c64", 1, 2, 150, 64),
    ("bf16", 1, 2, 200, 64),
    ("bf16", 1, 1, 77, 20),
    ("c64", 1, 1, 1, 8),
    # bf16 at width 64 runs on the matrix cores: several heads, ragged stages
    ("bf16", 2, 3, 333, 64),
    ("bf16", 1, 1, 65, 64),
    ("bf16", 1, 2, 1, 64),
    # complex64 at widths 16/32/64 runs on the fp32 matrix cores
    ("c64", 2, 3, 333, 64),
    ("c64", 1, 2, 100, 32),
    ("c64", 3, 1, 45, 16),
    # bf16 planes at widths 16/32 take the fp32 matrix-core kernels (widened on load)
    ("bf16", 2, 3, 333, 32),
    ("bf16", 1, 2, 100, 16),
]


@pytest.mark.parametrize("layout,B,H,T,d", STATE_CASES)
def test_state_build_and_accumulate(layout, B, H, T, d):
    from complex_valued_attention_amd import cattn
    w = gen.Workload("lin", "born", True, B, H, T, d, layout, seed=71)
    inp = gen.make_inputs(w)
    _, k, v = to_device(inp)
    say(f"state {layout} B{B} H{H} T{T} d{d}")
    S = cattn.born_state_buffer(B, H, d)
    S.fill_(float("nan"))   # overwrite mode ignores the old contents
    cattn.born_state(k, v, S)
    torch.cuda.synchronize()
    Sr = _oracle_state(inp, B, H, 0, T)
    err = _state_err(S, Sr)
    say(f"  full: {err:.3e}")
    assert err <= state_tol(layout, d)
    # the same state in two calls: overwrite (an empty first part zeroes the
    # state), then accumulate
    t1 = T // 3
    cattn.born_state(_slice(k, 0, t1), _slice(v, 0, t1), S)
    cattn.born_state(_slice(k, t1, T), _slice(v, t1, T), S, accumulate=True)
    torch.cuda.synchronize()
    err = _state_err(S, Sr)
    say(f"  split at {t1}: {err:.3e}")
    assert err <= state_tol(layout, d)


CARRY_CASES = [
    # (layout, B, H, T, T1, d, eps)
    ("c64", 1, 2, 300, 129, 64, 0.0),
    ("c64", 2, 1, 200, 64, 16, 0.0),
    ("c64", 1, 1, 150, 70, 33, 0.5),
    ("bf16", 1, 2, 300, 100, 64, 0.0),
    ("bf16", 1, 1, 90, 1, 32, 0.0),
    ("c64", 1, 1, 65, 64, 64, 0.0),     # one-token second call
    # bf16 at width 64 runs on the matrix cores: several 256-token tiles with
    # ragged tails; 24 workgroups (the XCD-grouped order) and 3 (plain order)
    ("bf16", 2, 3, 1100, 300, 64, 0.0),
    ("bf16", 1, 1, 700, 129, 64, 0.25),
    ("c64", 2, 3, 700, 300, 64, 0.0),
    ("c64", 1, 2, 333, 100, 32, 0.25),
    ("c64", 2, 2, 150, 17, 16, 0.0),
    ("bf16", 1, 2, 333, 100, 32, 0.25),
    ("bf16", 2, 2, 150, 17, 16, 0.0),
]


@pytest.mark.parametrize("layout,B,H,T,T1,d,eps", CARRY_CASES)
def test_prefill_with_carried_state(layout, B, H, T, T1, d, eps):
    """Tokens [0, T1) carried as a state, [T1, T) run as a causal forward and
    merged: equals causal Born over the whole sequence on [T1, T)."""
    import oracle
    from complex_valued_attention_amd import cattn
    w = gen.Workload("carry", "born", True, B, H, T, d, layout, seed=72, qk_unit=True)
    inp = gen.make_inputs(w)
    q, k, v = to_device(inp)
    say(f"carry {layout} B{B} H{H} T{T} split {T1} d{d} eps {eps}")
    S = cattn.born_state_buffer(B, H, d)
    cattn.born_state(_slice(k, 0, T1), _slice(v, 0, T1), S)
    q2, k2, v2 = (_slice(x, T1, T) for x in (q, k, v))
    row_den = torch.empty(B * H * (T - T1), dtype=torch.float32, device="cuda")
    o2 = cattn.born_fwd(q2, k2, v2, causal=True, eps=eps, row_den=row_den)
    cattn.born_merge(q2, S, o2, row_den)
    cattn.born_state(k2, v2, S, accumulate=True)
    torch.cuda.synchronize()
    ref = oracle.born_attention(inp.q64, inp.k64, inp.v64, causal=True, eps=eps)[:, :, T1:]
    err = rowwise_rel_err(from_device(o2), ref)
    say(f"  output: {err:.3e}")
    assert err <= TOL[layout]
    # merged row denominators are the full sequence's l = sum_j w + eps
    scores = np.einsum("bhtm,bhjm->bhtj", inp.q64, inp.k64.conj())
    w_ = np.abs(scores) ** 2
    l_ref = np.array([[[w_[b, h, t, : t + 1].sum() for t in range(T1, T)] for h in range(H)] for b in range(B)])
    l_ref = l_ref + eps
    l_got = row_den.cpu().numpy().reshape(B, H, T - T1)
    den_err = np.max(np.abs(l_got - l_ref) / l_ref)
    say(f"  row_den: {den_err:.3e}")
    assert den_err <= DEN_TOL[layout]
    assert _state_err(S, _oracle_state(inp, B, H, 0, T)) <= state_tol(layout, d)


STEP_CASES = [
    # (layout, B, H, T_prefix, steps, d, eps)
    ("c64", 1, 2, 0, 24, 64, 0.0),
    ("c64", 2, 1, 0, 20, 16, 0.25),
    ("c64", 1, 1, 100, 12, 33, 0.0),
    ("bf16", 1, 2, 0, 16, 64, 0.0),
    ("bf16", 1, 1, 50, 10, 20, 0.0),
]


@pytest.mark.parametrize("layout,B,H,T0,n,d,eps", STEP_CASES)
def test_step_decoding(layout, B, H, T0, n, d, eps):
    """Token-by-token decoding from a state (zero, or a prefix's) reproduces
    causal Born rows of the whole sequence."""
    import oracle
    from complex_valued_attention_amd import cattn
    T = T0 + n
    w = gen.Workload("step", "born", True, B, H, T, d, layout, seed=73)
    inp = gen.make_inputs(w)
    q, k, v = to_device(inp)
    say(f"step {layout} B{B} H{H} prefix {T0} steps {n} d{d} eps {eps}")
    S = cattn.born_state_buffer(B, H, d)
    if T0:
        cattn.born_state(_slice(k, 0, T0), _slice(v, 0, T0), S)
    outs, dens = [], []
    for t in range(T0, T):
        o, den = cattn.born_step(*(_slice(x, t, t + 1) for x in (q, k, v)), S, eps=eps)
        outs.append(from_device(o))
        dens.append(den.cpu().numpy().reshape(B, H))
    torch.cuda.synchronize()
    got = np.concatenate(outs, axis=2)
    ref = oracle.born_attention(inp.q64, inp.k64, inp.v64, causal=True, eps=eps)[:, :, T0:]
    err = rowwise_rel_err(got, ref)
    say(f"  outputs: {err:.3e}")
    assert err <= TOL[layout]
    # the oracle's own step recursion agrees on the denominators
    for b in range(B):
        for h in range(H):
            Zb, Mb = oracle.born_state(inp.k64[b, h, :T0], inp.v64[b, h, :T0])
            _, Zb, Mb = oracle.born_prefill(inp.q64[b, h, T0:], inp.k64[b, h, T0:], inp.v64[b, h, T0:], Zb, Mb, eps)
            q_last = inp.q64[b, h, T - 1]
            den_ref = (q_last.conj() @ Zb @ q_last).real + eps
            assert abs(dens[-1][b, h] - den_ref) <= 1e-4 * den_ref
    assert _state_err(S, _oracle_state(inp, B, H, 0, T)) <= state_tol(layout, d)


def test_step_zero_query_gives_zero():
    """q = 0 and eps = 0: the denominator is 0 and the output is 0 (the
    oracle's reading of an empty distribution)."""
    from complex_valued_attention_amd import cattn
    B, H, d = 1, 2, 16
    w = gen.Workload("z", "born", True, B, H, 1, d, "c64", seed=74)
    inp = gen.make_inputs(w)
    _, k, v = to_device(inp)
    q = torch.zeros_like(k)
    S = cattn.born_state_buffer(B, H, d)
    o, den = cattn.born_step(q, k, v, S, eps=0.0)
    torch.cuda.synchronize()
    assert torch.all(den == 0)
    assert torch.all(o == 0)


def test_step_at_full_head_count_sampled():
    """The step at 128 heads of width 64 after a 4096-token prefix (the state
    the decode measurement uses), checked on sampled heads against the oracle."""
    import oracle
    from complex_valued_attention_amd import cattn
    B, H, T0, d = 8, 16, 4096, 64
    w = gen.Workload("stepbig", "born", True, B, H, T0 + 1, d, "bf16", seed=3)
    inp = gen.make_inputs(w)
    q, k, v = to_device(inp)
    say(f"step full size B{B} H{H} prefix {T0} d{d} bf16")
    S = cattn.born_state_buffer(B, H, d)
    cattn.born_state(_slice(k, 0, T0), _slice(v, 0, T0), S)
    o, den = cattn.born_step(*(_slice(x, T0, T0 + 1) for x in (q, k, v)), S)
    torch.cuda.synchronize()
    got = from_device(o)
    for b, h in [(0, 0), (5, 11), (7, 15)]:
        Zb, Mb = oracle.born_state(inp.k64[b, h, :T0], inp.v64[b, h, :T0])
        ob, Zb, Mb = oracle.born_step(inp.q64[b, h, T0], inp.k64[b, h, T0], inp.v64[b, h, T0], Zb, Mb)
        err = rowwise_rel_err(got[b, h, 0][None], ob[None])
        es = _state_err(S[b, h], oracle.pack_state(Zb, Mb))
        say(f"  head ({b},{h}): out {err:.3e} state {es:.3e}")
        assert err <= TOL["bf16"]
        assert es <= state_tol("bf16", d)


@pytest.mark.parametrize("B,H,T,T1,d", [(2, 16, 2200, 152, 64), (4, 16, 1100, 76, 16), (2, 16, 2100, 50, 32)])
def test_prefill_with_carried_state_wide_sampled(B, H, T, T1, d):
    """A carried-state prefill with enough heads and chunk tokens that the
    complex64 readout takes its 128-token workgroups (the short-chunk tests
    take the 32-token ones): sampled rows of every head against the oracle's
    causal Born over the whole sequence."""
    import oracle
    from complex_valued_attention_amd import cattn
    w = gen.Workload("carrywide", "born", True, B, H, T, d, "c64", seed=74, qk_unit=True)
    inp = gen.make_inputs(w)
    q, k, v = to_device(inp)
    say(f"carry wide c64 B{B} H{H} T{T} split {T1} d{d}")
    S = cattn.born_state_buffer(B, H, d)
    cattn.born_state(_slice(k, 0, T1), _slice(v, 0, T1), S)
    q2, k2, v2 = (_slice(x, T1, T) for x in (q, k, v))
    row_den = torch.empty(B * H * (T - T1), dtype=torch.float32, device="cuda")
    o2 = cattn.born_fwd(q2, k2, v2, causal=True, row_den=row_den)
    cattn.born_merge(q2, S, o2, row_den)
    torch.cuda.synchronize()
    got = from_device(o2)
    rng = np.random.default_rng(7)
    ts = np.concatenate([[0, 1, 127, 128, T - T1 - 1], rng.integers(0, T - T1, 11)])
    rows = np.array([(b, h, t) for b in range(B) for h in range(H) for t in ts])
    ref = oracle.born_attention_rows(inp.q64, inp.k64, inp.v64, rows + np.array([0, 0, T1]), causal=True)
    sel = got[rows[:, 0], rows[:, 1], rows[:, 2]]
    err = rowwise_rel_err(sel, ref)
    say(f"  {len(rows)} sampled rows: {err:.3e}")
    assert err <= TOL["c64"]
