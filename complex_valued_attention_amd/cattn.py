"""Python binding of libcattn (ctypes): argument marshalling only.

Every step of the forward and backward runs in the HIP kernels behind the C ABI
(``include/cattn.h``); PyTorch provides device memory and the current stream.
There is no fallback: if the library is not built, calls raise.

Tensors are ``[B, H, T, d_h]`` on one ROCm device:

* complex64: ``q, k, v`` are ``torch.complex64`` tensors;
* bf16 planes: ``q, k, v`` are ``(re, im)`` pairs of ``torch.bfloat16`` tensors.

Born options: ``decay`` (one gamma in (0, 1] per head, causal only: the
weight of key j for query k is gamma^(k - j) |<q_k, k_j>|^2, and the carried
state advances as Z <- gamma Z + k k^H) is accepted by the Born forward,
backward and carried-state calls; the forward also rotates Q at load when
given ``rotary_base`` (K is then expected already rotated).

The forward calls take strided views (the last dimension contiguous, the two
planes of a pair with equal strides), e.g. slices of one fused projection
output; their strides go to the library as they are.  The backward, rotary
and carried-state calls take contiguous tensors.  The output has the layout of
the inputs.
"""
from __future__ import annotations

import ctypes
import math
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_lib", "libcattn.so")

LAYOUT_C64 = 0
LAYOUT_BF16_PLANES = 1

STATUS = {
    0: "CATTN_OK", 1: "CATTN_E_NULL", 2: "CATTN_E_SHAPE", 3: "CATTN_E_LAYOUT", 4: "CATTN_E_ALIGN",
    5: "CATTN_E_ALIAS", 6: "CATTN_E_UNSUPPORTED", 7: "CATTN_E_LAUNCH", 8: "CATTN_E_ARG",
}

_lib = None


class Stride(ctypes.Structure):
    """cattn_stride: element strides of the batch, head and token dimensions."""
    _fields_ = [("b", ctypes.c_int64), ("h", ctypes.c_int64), ("t", ctypes.c_int64)]


class Strides(ctypes.Structure):
    """cattn_strides: the strides of Q, K, V and O of a forward call."""
    _fields_ = [("q", Stride), ("k", Stride), ("v", Stride), ("o", Stride)]


class BornOpts(ctypes.Structure):
    """cattn_born_opts: decay table (host float[H] or NULL) and rotary Q options."""
    _fields_ = [("decay", ctypes.POINTER(ctypes.c_float)), ("rotary_base", ctypes.c_float),
                ("rotary_pos0", ctypes.c_int64)]


class CattnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded libcattn.so, with argument types declared."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libcattn.so is not built ({LIB_PATH}); run "
                           "`python -m complex_valued_attention_amd.build` or __graft_entry__.build()")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    sp = ctypes.POINTER(Strides)
    fp = ctypes.POINTER(ctypes.c_float)
    L.cattn_born_fwd.argtypes = [ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, sp,
                                 ctypes.c_int, ctypes.c_float, vp, ctypes.POINTER(BornOpts), vp]
    L.cattn_born_fwd.restype = ctypes.c_int
    L.cattn_pct_fwd.argtypes = [ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, sp,
                                ctypes.c_int, ctypes.c_float, vp]
    L.cattn_pct_fwd.restype = ctypes.c_int
    L.cattn_pct_gate_fwd.argtypes = [ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, sp,
                                     ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_float, vp]
    L.cattn_pct_gate_fwd.restype = ctypes.c_int
    L.cattn_rotary.argtypes = [ctypes.c_int, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_float, vp]
    L.cattn_rotary.restype = ctypes.c_int
    L.cattn_born_state.argtypes = [ctypes.c_int, vp, vp, vp, vp, i64, i64, i64, i64, vp, ctypes.c_int, fp, vp]
    L.cattn_born_state.restype = ctypes.c_int
    L.cattn_born_merge.argtypes = [ctypes.c_int, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, fp, vp]
    L.cattn_born_merge.restype = ctypes.c_int
    L.cattn_born_step.argtypes = [ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64,
                                  ctypes.c_float, fp, vp]
    L.cattn_born_step.restype = ctypes.c_int
    L.cattn_born_bwd.argtypes = [ctypes.c_int] + [vp] * 10 + [vp] + [vp] * 6 + [i64] * 4 + [ctypes.c_int, fp, vp]
    L.cattn_born_bwd.restype = ctypes.c_int
    L.cattn_pct_bwd.argtypes = ([ctypes.c_int] + [vp] * 8 + [vp] * 6 + [i64] * 4 +
                                [ctypes.c_int, ctypes.c_float, vp, vp])
    L.cattn_pct_bwd.restype = ctypes.c_int
    L.cattn_status_str.argtypes = [ctypes.c_int]
    L.cattn_status_str.restype = ctypes.c_char_p
    L.cattn_abi_version.argtypes = []
    L.cattn_abi_version.restype = ctypes.c_int
    _lib = L
    return L


def status_str(s: int) -> str:
    return lib().cattn_status_str(s).decode()


def _check(s: int):
    if s != 0:
        raise CattnError(s, status_str(s))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _unpack(x, name, strided=False):
    """(layout, re, im, shape) of one operand.  A strided operand needs only a
    contiguous last dimension (and equal strides on both planes); otherwise the
    tensors must be contiguous."""
    import torch

    def ok(t):
        if not t.is_cuda:
            raise ValueError(f"{name}: device tensors expected")
        if strided:
            if t.dim() != 4 or (t.shape[-1] > 1 and t.stride(-1) != 1):
                raise ValueError(f"{name}: [B, H, T, d_h] with a contiguous last dimension expected")
        elif not t.is_contiguous():
            raise ValueError(f"{name}: contiguous device tensors expected")

    if isinstance(x, (tuple, list)):
        re, im = x
        if re.dtype != torch.bfloat16 or im.dtype != torch.bfloat16:
            raise TypeError(f"{name}: bf16 planes expected")
        if re.shape != im.shape:
            raise ValueError(f"{name}: real and imaginary planes differ in shape")
        if re.device != im.device:
            raise ValueError(f"{name}: real and imaginary planes on different devices")
        ok(re)
        ok(im)
        if strided and re.stride() != im.stride():
            raise ValueError(f"{name}: real and imaginary planes differ in strides")
        return LAYOUT_BF16_PLANES, re, im, tuple(re.shape)
    if x.dtype != torch.complex64:
        raise TypeError(f"{name}: torch.complex64 or a (re, im) pair of bf16 tensors expected")
    ok(x)
    return LAYOUT_C64, x, None, tuple(x.shape)


def _stride3(t, name):
    """cattn_stride of a [B, H, T, d_h] tensor (elements).  The C ABI reads a
    zero stride as the dense value, so a broadcast view (stride 0 on a
    dimension longer than 1) is refused rather than misread."""
    for n, st in zip(t.shape[:3], t.stride()[:3]):
        if n > 1 and st == 0:
            raise ValueError(f"{name}: broadcast (zero-stride) views are not supported; pass a materialised tensor")
    sb, sh, st, _ = t.stride()
    return Stride(sb, sh, st)


def _prepare(q, k, v, out, strided=False):
    """Layout, the eight plane pointers' tensors, the shape, the output and
    (strided calls) the cattn_strides to pass, or None when all are dense."""
    import torch
    lq, qre, qim, shape = _unpack(q, "q", strided)
    lk, kre, kim, sk = _unpack(k, "k", strided)
    lv, vre, vim, sv = _unpack(v, "v", strided)
    if not (lq == lk == lv):
        raise TypeError("q, k and v must share one layout")
    if not (shape == sk == sv) or len(shape) != 4:
        raise ValueError(f"q, k, v must all be [B, H, T, d_h]; got {shape}, {sk}, {sv}")
    if not (qre.device == kre.device == vre.device):
        raise ValueError("q, k and v must be on one device")
    if out is None:
        if lq == LAYOUT_C64:
            out = torch.empty(shape, dtype=torch.complex64, device=qre.device)
        else:
            out = tuple(torch.empty(shape, dtype=torch.bfloat16, device=qre.device) for _ in range(2))
    lo, ore, oim, so = _unpack(out, "out", strided)
    if lo != lq or so != shape:
        raise ValueError("out must match the inputs' layout and shape")
    if ore.device != qre.device:
        raise ValueError("out must be on the inputs' device")
    strides = None
    if strided and not all(t.is_contiguous() for t in (qre, kre, vre, ore)):
        strides = Strides(_stride3(qre, "q"), _stride3(kre, "k"), _stride3(vre, "v"), _stride3(ore, "out"))
    return lq, (qre, qim, kre, kim, vre, vim, ore, oim), shape, out, strides


def _rows_f32(t, n, device, name):
    """Pointer of a per-row float32 buffer after checking it: float32,
    contiguous, ``n`` elements, on ``device`` (the inputs' device)."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: a torch.float32 tensor expected")
    if t.dtype != torch.float32:
        raise TypeError(f"{name}: torch.float32 expected, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name}: must be on {device}, got {t.device}")
    if not t.is_contiguous() or t.numel() != n:
        raise ValueError(f"{name}: a contiguous tensor of {n} elements expected")
    return _ptr(t)


def _stream(t):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _sref(strides):
    return None if strides is None else ctypes.byref(strides)


def _decay(decay, H):
    """A host float array of the H per-head decay values, or None."""
    if decay is None:
        return None
    try:
        import torch
        if isinstance(decay, torch.Tensor):
            decay = decay.detach().cpu().double().reshape(-1).tolist()
    except ImportError:
        pass
    vals = [float(x) for x in (decay if hasattr(decay, "__len__") else [decay] * H)]
    if len(vals) != H:
        raise ValueError(f"decay must hold one value per head ({H}), got {len(vals)}")
    return (ctypes.c_float * max(H, 1))(*vals)


def born_fwd(q, k, v, causal: bool = True, eps: float = 0.0, out=None, row_den=None, decay=None,
             rotary_base: float = 0.0, rotary_pos0: int = 0):
    """Born-rule attention forward (cattn_born_fwd).  Returns the output tensor(s).
    ``row_den`` (optional, float32 [B*H*T] on the inputs' device) receives the
    row denominators.  ``decay``: None, one gamma per head (a sequence or a
    tensor) or one gamma for all heads; ``rotary_base`` > 0 rotates Q at load
    from absolute position ``rotary_pos0``."""
    layout, ts, (B, H, T, d), out, strides = _prepare(q, k, v, out, strided=True)
    rd = None if row_den is None else _rows_f32(row_den, B * H * T, ts[0].device, "row_den")
    dec = _decay(decay, H)
    opts = None
    if dec is not None or rotary_base:
        opts = BornOpts(ctypes.cast(dec, ctypes.POINTER(ctypes.c_float)) if dec is not None else None,
                        float(rotary_base), int(rotary_pos0))
    s = lib().cattn_born_fwd(layout, *[_ptr(t) for t in ts], B, H, T, d, _sref(strides), int(bool(causal)),
                             float(eps), rd, None if opts is None else ctypes.byref(opts), _stream(ts[0]))
    _check(s)
    return out


def pct_fwd(q, k, v, causal: bool = False, bias: float = 0.0, out=None):
    """Phase-coherent attention forward (cattn_pct_fwd).  Returns the output tensor(s)."""
    layout, ts, (B, H, T, d), out, strides = _prepare(q, k, v, out, strided=True)
    s = lib().cattn_pct_fwd(layout, *[_ptr(t) for t in ts], B, H, T, d, _sref(strides), int(bool(causal)),
                            float(bias), _stream(ts[0]))
    _check(s)
    return out


GATES = {"sigmoid": 0, "softmax": 1, "screen": 2}


def pct_gate_fwd(q, k, v, gate: str = "softmax", causal: bool = False, a: float = 0.0, b: float = 0.0, out=None):
    """PCT-family forward with a chosen gate (cattn_pct_gate_fwd): "sigmoid" (bias a),
    "softmax" (the L2-softmax cell) or "screen" (a^2 max(s - b, 0)^2)."""
    if gate not in GATES:
        raise ValueError(f"gate must be one of {sorted(GATES)}")
    layout, ts, (B, H, T, d), out, strides = _prepare(q, k, v, out, strided=True)
    s = lib().cattn_pct_gate_fwd(layout, *[_ptr(t) for t in ts], B, H, T, d, _sref(strides), int(bool(causal)),
                                 GATES[gate], float(a), float(b), _stream(ts[0]))
    _check(s)
    return out


def rotary(x, pos0: int = 0, base: float = 10000.0, out=None):
    """Rotary phase embedding (cattn_rotary): x[..., t, m] * exp(i (pos0 + t) base^(-m/d_h)).
    ``out=x`` rotates in place.  Returns the output tensor(s)."""
    layout, re, im, shape = _unpack(x, "x")
    if len(shape) != 4:
        raise ValueError(f"x must be [B, H, T, d_h]; got {shape}")
    if out is None:
        out = _like(x)
    lo, ore, oim, so = _unpack(out, "out")
    if lo != layout or so != shape:
        raise ValueError("out must match x's layout and shape")
    B, H, T, d = shape
    s = lib().cattn_rotary(layout, _ptr(re), _ptr(im), _ptr(ore), _ptr(oim), B, H, T, d, int(pos0), float(base),
                           _stream(re))
    _check(s)
    return out


def born_state_buffer(B: int, H: int, d: int, device="cuda"):
    """A zeroed packed carried state: float32 [B, H, 2d + 1, d, d]."""
    import torch
    return torch.zeros(B, H, 2 * d + 1, d, d, dtype=torch.float32, device=device)


def _state_ptr(S, B, H, d, device):
    import torch
    if not isinstance(S, torch.Tensor) or S.dtype != torch.float32:
        raise TypeError("the state must be a torch.float32 tensor")
    if S.device != device:
        raise ValueError(f"the state must be on {device}, got {S.device}")
    if not S.is_contiguous() or tuple(S.shape) != (B, H, 2 * d + 1, d, d):
        raise ValueError("the state must be a contiguous float32 tensor [B, H, 2d + 1, d, d]")
    return _ptr(S)


def born_state(k, v, S, accumulate: bool = False, decay=None):
    """cattn_born_state: the packed state of the tokens of k, v (added to S's contents if accumulate;
    under ``decay`` the old contents first scale by gamma^T)."""
    lk, kre, kim, shape = _unpack(k, "k")
    lv, vre, vim, sv = _unpack(v, "v")
    if lk != lv or shape != sv or len(shape) != 4:
        raise ValueError("k and v must share a layout and a [B, H, T, d] shape")
    if kre.device != vre.device:
        raise ValueError("k and v must be on one device")
    B, H, T, d = shape
    _check(lib().cattn_born_state(lk, _ptr(kre), _ptr(kim), _ptr(vre), _ptr(vim), B, H, T, d,
                                  _state_ptr(S, B, H, d, kre.device), int(bool(accumulate)), _decay(decay, H),
                                  _stream(kre)))
    return S


def born_merge(q, S, o, row_den, decay=None):
    """cattn_born_merge: fold the incoming state S into a causal forward's o and row_den, in place
    (under ``decay`` the state counts gamma^(t+1) at token t)."""
    lq, qre, qim, shape = _unpack(q, "q")
    lo, ore, oim, so = _unpack(o, "o")
    if lq != lo or shape != so or len(shape) != 4:
        raise ValueError("q and o must share a layout and a [B, H, T, d] shape")
    if qre.device != ore.device:
        raise ValueError("q and o must be on one device")
    B, H, T, d = shape
    rd = _rows_f32(row_den, B * H * T, qre.device, "row_den")
    _check(lib().cattn_born_merge(lq, _ptr(qre), _ptr(qim), _state_ptr(S, B, H, d, qre.device), _ptr(ore),
                                  _ptr(oim), rd, B, H, T, d, _decay(decay, H), _stream(qre)))
    return o, row_den


def born_step(q, k, v, S, eps: float = 0.0, out=None, row_den=None, decay=None):
    """cattn_born_step: one token per head ([B, H, 1, d]); updates S in place (scaled by gamma first
    under ``decay``), returns (o, row_den)."""
    import torch
    layout, ts, (B, H, T, d), out, _ = _prepare(q, k, v, out)
    if T != 1:
        raise ValueError("born_step takes one token per head: [B, H, 1, d]")
    if row_den is None:
        row_den = torch.empty(B * H, dtype=torch.float32, device=ts[0].device)
    rd = _rows_f32(row_den, B * H, ts[0].device, "row_den")
    _check(lib().cattn_born_step(layout, *[_ptr(t) for t in ts], _state_ptr(S, B, H, d, ts[0].device), rd, B, H,
                                 d, float(eps), _decay(decay, H), _stream(ts[0])))
    return out, row_den


def _like(x):
    import torch
    if isinstance(x, (tuple, list)):
        return (torch.empty_like(x[0]), torch.empty_like(x[1]))
    return torch.empty_like(x)


def _same(x, ref, name):
    """(re, im) tensors of x after checking it matches ref's layout, shape and device."""
    lx, re, im, sx = _unpack(x, name)
    lr, rre, _, sr = _unpack(ref, "q")
    if lx != lr or sx != sr:
        raise ValueError(f"{name} must match q's layout and shape")
    if re.device != rre.device:
        raise ValueError(f"{name} must be on q's device")
    return re, im


def _bwd_outs(q, grads):
    if grads is None:
        grads = (_like(q), _like(q), _like(q))
    dq, dk, dv = grads
    return grads, [t for g, n in zip((dq, dk, dv), ("dq", "dk", "dv")) for t in _same(g, q, n)]


def born_bwd(q, k, v, o, g, row_den, causal: bool = True, grads=None, decay=None):
    """Born-rule attention backward (cattn_born_bwd).

    ``o`` and ``row_den`` come from the forward (``born_fwd(..., row_den=...)``);
    ``g`` is dL/d(conj O) (or the real-pair gradient, which gives real-pair
    gradients back).  ``decay`` is the forward's.  Returns ``(dq, dk, dv)``
    in the inputs' layout.
    """
    layout, ts, (B, H, T, d), _, _ = _prepare(q, k, v, _like(q))
    ore, oim = _same(o, q, "o")
    gre, gim = _same(g, q, "g")
    if row_den is None:
        raise ValueError("row_den (the forward's row denominators) is required")
    rd = _rows_f32(row_den, B * H * T, ts[0].device, "row_den")
    grads, outs = _bwd_outs(q, grads)
    s = lib().cattn_born_bwd(layout, *[_ptr(t) for t in ts[:6]], _ptr(ore), _ptr(oim), _ptr(gre), _ptr(gim),
                             rd, *[_ptr(t) for t in outs], B, H, T, d, int(bool(causal)), _decay(decay, H),
                             _stream(ts[0]))
    _check(s)
    return grads


def pct_bwd(q, k, v, g, causal: bool = False, bias: float = 0.0, grads=None, db_rows=None):
    """Phase-coherent attention backward (cattn_pct_bwd).  Returns ``(dq, dk, dv)``;
    ``db_rows`` (optional float32 [B*H*T]) receives the per-row bias gradient."""
    layout, ts, (B, H, T, d), _, _ = _prepare(q, k, v, _like(q))
    gre, gim = _same(g, q, "g")
    db = None if db_rows is None else _rows_f32(db_rows, B * H * T, ts[0].device, "db_rows")
    grads, outs = _bwd_outs(q, grads)
    s = lib().cattn_pct_bwd(layout, *[_ptr(t) for t in ts[:6]], _ptr(gre), _ptr(gim),
                            *[_ptr(t) for t in outs], B, H, T, d, int(bool(causal)), float(bias),
                            db, _stream(ts[0]))
    _check(s)
    return grads


def default_pct_bias(T: int) -> float:
    """The pages' initial gate bias -log N."""
    return -math.log(T)
