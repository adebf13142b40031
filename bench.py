"""Benchmark: Born-rule attention forward, B8 H16 T4096 d_h 64, bf16 real/imag planes.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline] [--copy-probe MIB]
    python bench.py --pass bwd [--workload NAME] ...      (the backward instead of the forward)
    python bench.py --workload NAME --gate softmax|screen  (a PCT workload with a sibling gate)
    python bench.py --pass step [--workload NAME]        (one-token decoding with a carried Born state)
    python bench.py --pass linear [--workload NAME] [--chunk C]
                                   (a whole causal Born sequence in chunks with a carried state, beside
                                    the quadratic kernel on the same inputs)

One step = one call of the fused forward (score GEMM, weight map, Born
denominator, value GEMM, epilogue: the whole hot path, one kernel launch)
over one batch of synthetic inputs already resident in HBM.  Prints ONE JSON
line on stdout: the throughput in real TFLOP/s (8 T^2 d_h for S plus
4 T^2 d_h for W V per head, halved for causal attention), the roofline of
the kernel measured with HIP events on the launch stream, and the fp64 oracle
timed on a bounded sample of whole heads on the host cores as a CPU baseline
(its heads are also compared with the GPU output).
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Born-attn fwd real TFLOP/s (B8 H16 T4096 d64) + % MFMA peak"
# MI355X published dense peaks (TFLOP/s) and HBM bandwidth (GB/s)
PEAK_TFLOPS = {"bf16": 2500.0, "c64": 157.3}
PEAK_HBM_GBS = 8000.0

# HBM bytes per launch of the dominant kernel, from two rocprofv3 passes
# (FETCH_SIZE, then WRITE_SIZE) scaled by what the same counters read for the
# --copy-probe kernel.  Valid only for the kernel source it was measured on:
# any other source gives traffic = null.
MEASURED_TRAFFIC = {
    # name -> {"source": kernel file, "sha256": its hash when the counters were
    # taken, "bytes": FETCH_SIZE + WRITE_SIZE per launch, scaled by the copy probe}
    "born_causal_bf16_b8h16t4096d64_rotary": {
        "source": "complex_valued_attention_amd/csrc/kernel_born_bf16_d64.hip",
        "sha256": "7c6c753ec257cb2bcb7994a9cefdb6a4d9be0ae4b53adfd20d83b712767e6259",
        "bytes": 930.9e6,   # read 796.7 MB + write 134.2 MB
    },
    # the bench workload's shape at head width 128 (bench.py --d-h 128)
    "born_causal_bf16_b8h16t4096d64_rotary@d128": {
        "source": "complex_valued_attention_amd/csrc/born_bf16_q16_impl.h",
        "sha256": "68eb1accd09ff91e97b784ae0e67cd3dccffb6158e3ba261555a07ebea288074",
        "bytes": 1706.9e6,  # read 1438.5 MB + write 268.4 MB
    },
    # the carried-state kernels of --pass linear at chunk 4096 (mean per launch over a pass)
    "linear-state:born_causal_bf16_b1h16t32768d64_rotary:4096": {
        "source": "complex_valued_attention_amd/csrc/kernel_born_linear_bf16.hip",
        "sha256": "edb94da4d42529beee88a404769fb38cbc9b91943c03cc8dbe8a342660201698",
        "bytes": 96.6e6,    # read 62.8 MB + write 33.8 MB
    },
    "linear-merge:born_causal_bf16_b1h16t32768d64_rotary:4096": {
        "source": "complex_valued_attention_amd/csrc/kernel_born_linear_bf16.hip",
        "sha256": "edb94da4d42529beee88a404769fb38cbc9b91943c03cc8dbe8a342660201698",
        "bytes": 85.4e6,    # read 67.9 MB + write 17.5 MB
    },
    # the whole backward call of --pass bwd (per-query scalars, dK/dV, dQ), per call
    "bwd:born_causal_bf16_b8h16t4096d64_rotary": {
        "source": "complex_valued_attention_amd/csrc/kernel_born_bf16_d64_bwd.hip",
        "sha256": "3a47f8b1fc6f43fd8f52a742cde89a6d31ccafbd70382cc973e98c163609ea1a",
        "bytes": 2153.9e6,  # read 270.8 + 561.6 + 876.9 MB, write 4.2 + 268.4 + 172.0 MB
    },
}


def measured_traffic(name: str):
    import hashlib
    m = MEASURED_TRAFFIC.get(name)
    if m is None:
        return None
    with open(os.path.join(ROOT, m["source"]), "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != m["sha256"]:
            return None
    return m["bytes"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_flops(w) -> float:
    """Flops the method needs: Born 12 d_h per (query, key) pair, PCT 8 d_h (only Re S)."""
    from complex_valued_attention_amd.inputs import attention_flops
    f = attention_flops(w.T, w.d_h, w.causal, w.B * w.H)
    return f if w.op == "born" else f * 8.0 / 12.0


def kernel_name(w) -> str:
    """The HIP kernel the library dispatches for this workload."""
    if w.op == "born" and w.layout == "bf16" and w.d_h in (16, 32, 64, 128):
        return {64: "born_bf16_d64_kernel", 128: "born_bf16_q16_kernel", 32: "born_bf16_q16_kernel"}.get(
            w.d_h, "born_bf16_mfma_kernel")
    if w.d_h in (16, 32, 64, 128):   # complex64, and PCT on bf16 planes
        return "attn_f32_mfma16_kernel"
    return "generic_fwd_kernel"


def bwd_flops(w) -> float:
    """Minimal backward flops: S, E = Re(G^H V), dV, dK and dQ once each -- Born
    (8 + 4 + 4 + 8 + 8) d_h = 32 d_h per (query, key) pair, PCT (4 + 4 + 4 + 4 + 4)
    d_h = 20 d_h (only Re S, real weights); halved when causal."""
    per_pair = 32.0 if w.op == "born" else 20.0
    f = per_pair * w.T * w.T * w.d_h * w.B * w.H
    return f / 2 if w.causal else f


def run_gpu_bwd(w, steps: int, warmup: int):
    """Times the backward call alone; O and the row denominators come from one
    forward call before the timed region."""
    import torch
    from complex_valued_attention_amd import cattn, inputs as gen
    from complex_valued_attention_amd.check import from_device, grad_to_device, to_device

    cattn.lib()
    inp = gen.make_inputs(w)
    grad = gen.make_grad(w)
    q, k, v = to_device(inp)
    g = grad_to_device(grad)
    like = (lambda: torch.empty_like(q)) if w.layout == "c64" else (lambda: (torch.empty_like(q[0]),
                                                                            torch.empty_like(q[0])))
    grads = (like(), like(), like())
    if w.op == "born":
        den = torch.empty(w.B * w.H * w.T, dtype=torch.float32, device="cuda")
        o = cattn.born_fwd(q, k, v, causal=w.causal, row_den=den)
        step = lambda: cattn.born_bwd(q, k, v, o, g, den, causal=w.causal, grads=grads)
    else:
        step = lambda: cattn.pct_bwd(q, k, v, g, causal=w.causal, grads=grads)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    return inp, grad, tuple(from_device(x) for x in grads), ev[0].elapsed_time(ev[-1]) / steps, per


def main_bwd(args, w):
    from complex_valued_attention_amd.check import rowwise_rel_err
    inp, grad, got, ms, per = run_gpu_bwd(w, args.steps, args.warmup)
    flops = bwd_flops(w)
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"[bench] bwd {w.name}: {ms:.4f} ms/step (median {np.median(per):.4f} ms), {tflops:.2f} TFLOP/s")
    # which kernels the library dispatches: bf16 matrix cores for Born at d_h = 64, fp32 matrix
    # cores for complex64 and bf16 planes otherwise (16 x 16 tiles at d_h 32/64/128, 32 x 32 at
    # 16), else fp32 vector code
    mfma = w.op == "born" and w.layout == "bf16" and w.d_h == 64
    mfma32 = not mfma and w.d_h in (16, 32, 64, 128)
    peak = PEAK_TFLOPS["bf16"] if mfma else PEAK_TFLOPS["c64"]
    kern = ("born_bf16_d64_bwd_dkdv_kernel + born_bf16_d64_bwd_dq_kernel" if mfma
            else "bwd16_dkdv_kernel + bwd16_dq_kernel" if w.d_h in (32, 64, 128)
            else "bwd_dkdv_f32_kernel + bwd_dq_f32_kernel" if mfma32
            else "bwd_dkdv_kernel + bwd_dq_kernel")
    rec = {
        "metric": f"{w.op} bwd real TFLOP/s ({w.name})",
        "value": tflops, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if mfma else "f32", "data": "synthetic",
        "config": {"workload": w.name, "pass": "bwd", "op": w.op, "causal": w.causal, "B": w.B, "H": w.H,
                   "T": w.T, "d_h": w.d_h, "layout": w.layout},
        "roofline": {"bound": "mfma" if (mfma or mfma32) else "alu", "achieved": tflops, "peak": peak, "unit": "TFLOP/s",
                     "frac": tflops / peak, "traffic": measured_traffic(f"bwd:{w.name}"), "kernel": kern},
    }
    if not args.no_cpu_baseline:
        import oracle
        from threadpoolctl import threadpool_info
        t0 = time.perf_counter()
        b, h = 0, 0
        if w.op == "born":
            ref = oracle.born_attention_bwd(inp.q64[b, h], inp.k64[b, h], inp.v64[b, h], grad.g64[b, h],
                                            causal=w.causal)
        else:
            ref = oracle.pct_attention_bwd(inp.q64[b, h], inp.k64[b, h], inp.v64[b, h], grad.g64[b, h],
                                           causal=w.causal)[:3]
        t = time.perf_counter() - t0
        one = dataclasses.replace(w, B=1, H=1)
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        rec["cpu_baseline"] = {"value": bwd_flops(one) / t / 1e12, "unit": "TFLOP/s", "cores": int(threads), **host_info(),
                               "kind": "oracle", "sample": f"1 of {w.B * w.H} heads (full T={w.T}), fp64 numpy, "
                                                           f"{t:.1f} s",
                               "gpu_rowwise_rel_err_dv": rowwise_rel_err(got[2][b, h], ref[2])}
    print(json.dumps(rec), flush=True)


def main_rotary(args, w):
    """The rotary pass over one [B, H, T, d_h] operand of the workload (out of place):
    HBM-bound, bytes = the operand read once + written once."""
    import torch
    from complex_valued_attention_amd import cattn
    from complex_valued_attention_amd.check import to_device
    cattn.lib()
    inp = __import__("complex_valued_attention_amd.inputs", fromlist=["make_inputs"]).make_inputs(w)
    x = to_device(inp)[0]
    out = cattn.rotary(x)
    for _ in range(args.warmup):
        cattn.rotary(x, out=out)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    ev[0].record(stream)
    for i in range(args.steps):
        cattn.rotary(x, out=out)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[-1]) / args.steps
    nbytes = 2 * w.B * w.H * w.T * w.d_h * (8 if w.layout == "c64" else 4)
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"[bench] rotary {w.name}: {ms:.4f} ms/step, {gbs:.0f} GB/s")
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        from threadpoolctl import threadpool_info
        from complex_valued_attention_amd.check import TOL, from_device, rowwise_rel_err
        got = from_device(out)
        done, t_used, err = 0, 0.0, 0.0
        for b in range(w.B):
            for h in range(w.H):
                t0 = time.perf_counter()
                ref = oracle.rotary(inp.q64[b, h][None, None])[0, 0]
                t_used += time.perf_counter() - t0
                err = max(err, rowwise_rel_err(got[b, h], ref))
                done += 1
                if t_used >= 12.0:
                    break
            if t_used >= 12.0:
                break
        per_head = 2 * w.T * w.d_h * (8 if w.layout == "c64" else 4)
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        cpu = {"value": done * per_head / t_used / 1e9, "unit": "GB/s", "cores": int(threads), **host_info(), "kind": "oracle",
               "sample": f"{done} of {w.B * w.H} heads of Q (full T={w.T}), fp64 numpy, {t_used:.1f} s",
               "gpu_rowwise_rel_err": err, "gpu_parity_pass": bool(err <= TOL[w.layout])}
    rec = {"metric": f"rotary GB/s ({w.name})", "value": gbs, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "f32" if w.layout == "c64" else "bf16", "data": "synthetic",
           "config": {"workload": w.name, "pass": "rotary", "B": w.B, "H": w.H, "T": w.T, "d_h": w.d_h,
                      "layout": w.layout},
           "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": gbs / PEAK_HBM_GBS, "traffic": None, "kernel": "rotary_kernel"}}
    if cpu is not None:
        rec["cpu_baseline"] = cpu
    print(json.dumps(rec), flush=True)


def _chunk(x, t0, t1):
    """[B, H, t0:t1, d] as a fresh contiguous allocation (complex64 tensor or bf16 plane pair)."""
    import torch
    if isinstance(x, tuple):
        return tuple(p[:, :, t0:t1].clone(memory_format=torch.contiguous_format) for p in x)
    return x[:, :, t0:t1].clone(memory_format=torch.contiguous_format)


def state_flops(T: int, d: int, heads: int) -> float:
    """Real flops of building (or reading out) the carried state over T tokens:
    2d + 1 packed real d x d matrices per head, one multiply-add per entry and
    token (forming the d^2 lifted features of a token is not counted)."""
    return 2.0 * T * (2 * d + 1) * d * d * heads


def state_bytes(d: int, heads: int) -> int:
    """Bytes of the packed carried state (fp32)."""
    return (2 * d + 1) * d * d * 4 * heads


def main_step(args, w):
    """One-token decoding with a carried Born state: the state of the workload's
    T tokens is built once (untimed), then each step adds one token and reads
    the state out.  HBM-bound: the state is read and written once per step."""
    import oracle
    import torch
    from complex_valued_attention_amd import cattn, inputs as gen
    from complex_valued_attention_amd.check import TOL, from_device, rowwise_rel_err, to_device
    from threadpoolctl import threadpool_info
    if w.op != "born" or w.d_h > 64:
        print("--pass step needs a Born workload with d_h <= 64", file=sys.stderr)
        sys.exit(2)
    cattn.lib()
    inp = gen.make_inputs(w)
    q, k, v = to_device(inp)
    B, H, T, d = w.B, w.H, w.T, w.d_h
    n = args.warmup + args.steps
    if n > T:
        print(f"--warmup + --steps must not exceed T = {T}", file=sys.stderr)
        sys.exit(2)
    S = cattn.born_state_buffer(B, H, d)
    cattn.born_state(k, v, S)
    # the new tokens: the workload's first n tokens again, one fresh [B, H, 1, d] tensor each
    toks = [tuple(_chunk(x, t, t + 1) for x in (q, k, v)) for t in range(n)]
    outs = [cattn._like(toks[0][0]) for _ in range(n)]
    dens = torch.empty(n, B * H, dtype=torch.float32, device="cuda")
    for i in range(args.warmup):
        cattn.born_step(*toks[i], S, out=outs[i], row_den=dens[i])
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    ev[0].record(stream)
    for i in range(args.warmup, n):
        cattn.born_step(*toks[i], S, out=outs[i], row_den=dens[i])
        ev[i - args.warmup + 1].record(stream)
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]
    ms = ev[0].elapsed_time(ev[-1]) / args.steps
    heads = B * H
    elem = 8 if w.layout == "c64" else 4
    nbytes = 2 * state_bytes(d, heads) + 4 * heads * d * elem + 4 * heads   # state in and out, q k v o, row_den
    gbs = nbytes / (float(np.mean(per)) * 1e-3) / 1e9
    log(f"[bench] step {w.name}: {ms:.4f} ms/step ({heads} heads, state {state_bytes(d, heads) / 2**20:.0f} MiB), "
        f"{gbs:.0f} GB/s")
    # oracle: head (0, 0) through the same T-token prefix and every step (its
    # outputs compared with the device's); then more steps on the workload's
    # tokens until about 12 s of host time, the CPU baseline
    b, h = 0, 0
    Zo, Mo = oracle.born_state(inp.k64[b, h], inp.v64[b, h])
    t_used, err, n_cpu = 0.0, 0.0, 0
    while n_cpu < n or (t_used < 12.0 and n_cpu < T):
        t0 = time.perf_counter()
        o_ref, Zo, Mo = oracle.born_step(inp.q64[b, h, n_cpu], inp.k64[b, h, n_cpu], inp.v64[b, h, n_cpu], Zo, Mo)
        t_used += time.perf_counter() - t0
        if n_cpu < n:
            err = max(err, rowwise_rel_err(from_device(outs[n_cpu])[b, h], o_ref[None]))
        n_cpu += 1
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    rec = {"metric": f"Born carried-state decode tokens/s ({w.name} state)", "value": heads / (ms * 1e-3),
           "unit": "head-tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "f32", "data": "synthetic (the workload's tokens as prefix and as new tokens)",
           "config": {"workload": w.name, "pass": "step", "B": B, "H": H, "prefix_T": T, "d_h": d,
                      "layout": w.layout, "state_MiB": state_bytes(d, heads) / 2**20},
           "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": gbs / PEAK_HBM_GBS, "traffic": measured_traffic(f"step:{w.name}"),
                        "kernel": "born_step_kernel",
                        "bytes_per_step": nbytes, "kernel_ms_mean": float(np.mean(per)),
                        "kernel_ms_median": float(np.median(per))},
           "cpu_baseline": {"value": n_cpu / t_used, "unit": "head-tokens/s", "cores": int(threads), **host_info(), "kind": "oracle",
                            "sample": f"head (0,0), {n_cpu} steps after the {T}-token prefix, fp64 numpy, "
                                      f"{t_used:.1f} s", "gpu_rowwise_rel_err": err,
                            "gpu_parity_pass": bool(err <= TOL[w.layout])}}
    print(json.dumps(rec), flush=True)


def main_linear(args, w):
    """A whole causal Born sequence in chunks of C tokens with a carried state:
    the quadratic kernel within each chunk, then per chunk the merge of the
    incoming state and the state update; beside it the quadratic kernel over
    the whole sequence on the same inputs.  The within-chunk products do not
    depend on the state, so when C divides T they run as one launch over all
    chunks (a strided view of the sequence as [chunks, B*H, C, d_h], the
    outputs chunk-major), which fills the chip where one chunk of few heads
    would not; otherwise one launch per chunk."""
    import oracle
    import torch
    from complex_valued_attention_amd import cattn, inputs as gen
    from complex_valued_attention_amd.check import TOL, from_device, rowwise_rel_err, sample_rows, to_device
    from threadpoolctl import threadpool_info
    if w.op != "born" or not w.causal or w.d_h > 64:
        print("--pass linear needs a causal Born workload with d_h <= 64", file=sys.stderr)
        sys.exit(2)
    cattn.lib()
    inp = gen.make_inputs(w)
    q, k, v = to_device(inp)
    B, H, T, d, C = w.B, w.H, w.T, w.d_h, args.chunk
    nc = (T + C - 1) // C
    chunks = [tuple(_chunk(x, i * C, min(T, (i + 1) * C)) for x in (q, k, v)) for i in range(nc)]
    batched = T % C == 0 and nc > 1
    if batched:
        # chunk-major views: operand element (c, b*H + h, t, :) is row c*C + t of head (b, h)
        def view(x):
            if isinstance(x, tuple):
                return tuple(view(p) for p in x)
            return x.as_strided((nc, B * H, C, d), (C * d, T * d, d, 1))
        qv, kv, vv = view(q), view(k), view(v)
        fresh = lambda x: torch.empty((nc, B * H, C, d), dtype=x.dtype, device=x.device)
        out_all = tuple(fresh(p) for p in qv) if isinstance(qv, tuple) else fresh(qv)
        den_all = torch.empty(nc * B * H * C, dtype=torch.float32, device="cuda")
        pick = lambda x, i: tuple(p[i].view(B, H, C, d) for p in x) if isinstance(x, tuple) else x[i].view(B, H, C, d)
        outs = [pick(out_all, i) for i in range(nc)]
        dens = [den_all[i * B * H * C:(i + 1) * B * H * C] for i in range(nc)]
    else:
        outs = [cattn._like(c[0]) for c in chunks]
        dens = [torch.empty(B * H * min(C, T - i * C), dtype=torch.float32, device="cuda") for i in range(nc)]
    S = cattn.born_state_buffer(B, H, d)
    stream = torch.cuda.current_stream()
    kinds = ("fwd", "merge", "state")

    def chunked(evs=None):
        if batched:
            marks = []
            if evs is not None:
                marks.append(torch.cuda.Event(enable_timing=True)); marks[-1].record(stream)
            cattn.born_fwd(qv, kv, vv, causal=True, out=out_all, row_den=den_all)
            if evs is not None:
                marks.append(torch.cuda.Event(enable_timing=True)); marks[-1].record(stream)
                evs.append(marks + [marks[-1], marks[-1]])
        for i, (qc, kc, vc) in enumerate(chunks):
            marks = []
            if evs is not None:
                marks.append(torch.cuda.Event(enable_timing=True)); marks[-1].record(stream)
            if not batched:
                cattn.born_fwd(qc, kc, vc, causal=True, out=outs[i], row_den=dens[i])
            if evs is not None:
                marks.append(torch.cuda.Event(enable_timing=True)); marks[-1].record(stream)
            if i:
                cattn.born_merge(qc, S, outs[i], dens[i])
            if evs is not None:
                marks.append(torch.cuda.Event(enable_timing=True)); marks[-1].record(stream)
            if i + 1 < nc:
                cattn.born_state(kc, vc, S, accumulate=i > 0)
            if evs is not None:
                marks.append(torch.cuda.Event(enable_timing=True)); marks[-1].record(stream)
                evs.append(marks)

    full_out = cattn._like(q)
    quad = lambda: cattn.born_fwd(q, k, v, causal=True, out=full_out)
    for _ in range(args.warmup):
        chunked()
        quad()
    torch.cuda.synchronize()
    # the chunked form, whole passes timed
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    ev[0].record(stream)
    for i in range(args.steps):
        chunked()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[-1]) / args.steps
    # per-kind kernel time (a separate pass with events between the launches)
    evs = []
    chunked(evs)
    torch.cuda.synchronize()
    part = {kd: sum(m[j].elapsed_time(m[j + 1]) for m in evs) for j, kd in enumerate(kinds)}
    # the quadratic kernel over the whole sequence
    eq = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    eq[0].record(stream)
    for i in range(args.steps):
        quad()
        eq[i + 1].record(stream)
    torch.cuda.synchronize()
    ms_quad = eq[0].elapsed_time(eq[-1]) / args.steps
    heads = B * H
    tok_s = heads * T / (ms * 1e-3)
    log(f"[bench] linear {w.name} chunk {C}: {ms:.3f} ms/pass ({tok_s / 1e6:.2f} M head-tokens/s); "
        f"quadratic {ms_quad:.3f} ms; parts {part}")
    # parity: the chunked output against the quadratic kernel's on every row,
    # and sampled rows against the oracle
    got = np.concatenate([from_device(o) for o in outs], axis=2)
    quad_got = from_device(full_out)
    err_quad = rowwise_rel_err(got, quad_got)
    rows = sample_rows(B, H, T, 32, seed=w.seed, tile=C)
    t0 = time.perf_counter()
    ref = oracle.born_attention_rows(inp.q64, inp.k64, inp.v64, rows, causal=True)
    t_rows = time.perf_counter() - t0
    err = rowwise_rel_err(got[rows[:, 0], rows[:, 1], rows[:, 2]], ref)
    # CPU baseline: the oracle's own carried-state recursion on the first tokens of head (0, 0)
    n_cpu, t_used = 0, 0.0
    Zo, Mo = np.zeros((d, d), complex), np.zeros((d, d, d), complex)
    while t_used < 12.0 and n_cpu < T:
        t0 = time.perf_counter()
        _, Zo, Mo = oracle.born_step(inp.q64[0, 0, n_cpu], inp.k64[0, 0, n_cpu], inp.v64[0, 0, n_cpu], Zo, Mo)
        t_used += time.perf_counter() - t0
        n_cpu += 1
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    dom = max(("merge", "state"), key=lambda kd: part[kd])
    n_launch = nc - 1
    dom_ms = part[dom] / n_launch
    dom_flops = state_flops(C, d, heads)
    achieved = dom_flops / (dom_ms * 1e-3) / 1e12
    # bf16 planes at width 64 run the state kernels on the bf16 matrix cores, complex64 at widths
    # 16/32/64 on the fp32 matrix cores; otherwise the fp32 vector ALU
    mfma = w.layout == "bf16" and d == 64
    mfma32 = w.layout == "c64" and d in (16, 32, 64)
    bound, peak = ("mfma", PEAK_TFLOPS["bf16"]) if mfma else ("mfma" if mfma32 else "alu", PEAK_TFLOPS["c64"])
    suffix = "_bf16_d64" if mfma else "_f32" if mfma32 else ""
    kname = f"born_{dom}{suffix}_kernel"
    rec = {"metric": f"Born chunked carried-state prefill head-tokens/s ({w.name}, chunk {C})",
           "value": tok_s, "unit": "head-tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16" if w.layout == "bf16" else "f32",
           "data": "synthetic (seeded complex Gaussian, unit-norm rotary Q/K)" if w.rotary else "synthetic",
           "config": {"workload": w.name, "pass": "linear", "B": B, "H": H, "T": T, "d_h": d, "layout": w.layout,
                      "chunk": C, "chunks": nc, "within_chunk": "one launch over all chunks" if batched
                      else "one launch per chunk"},
           "quadratic_ms": ms_quad, "speedup_vs_quadratic": ms_quad / ms,
           "parts_ms": part,
           "roofline": {"bound": bound, "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                        "frac": achieved / peak,
                        "traffic": measured_traffic(f"linear-{dom}:{w.name}:{C}"),
                        "kernel": kname, "kernel_ms_mean": dom_ms,
                        "flops_per_launch": dom_flops},
           "gpu_vs_quadratic_rowwise_rel_err": err_quad,
           "cpu_baseline": {"value": n_cpu / t_used, "unit": "head-tokens/s", "cores": int(threads), **host_info(),
                            "kind": "oracle",
                            "sample": f"head (0,0), first {n_cpu} tokens by the oracle's step recursion, "
                                      f"fp64 numpy, {t_used:.1f} s; {len(rows)} sampled rows by the quadratic "
                                      f"definition in {t_rows:.1f} s",
                            "gpu_rowwise_rel_err": err, "gpu_parity_pass": bool(err <= TOL[w.layout])}}
    print(json.dumps(rec), flush=True)


def run_gpu(w, steps: int, warmup: int, gate: str = "sigmoid", born_opts=None, inp=None):
    import torch
    from complex_valued_attention_amd import cattn, inputs as gen
    from complex_valued_attention_amd.check import from_device, to_device

    cattn.lib()  # fails loudly if the HIP library is not built
    if inp is None:
        t0 = time.time()
        inp = gen.make_inputs(w)
        log(f"[bench] inputs {w.name}: {time.time() - t0:.1f} s")
    q, k, v = to_device(inp)
    if w.layout == "c64":
        out = torch.empty_like(q)
    else:
        out = (torch.empty_like(q[0]), torch.empty_like(q[0]))
    if w.op == "born":
        step = lambda: cattn.born_fwd(q, k, v, causal=w.causal, out=out, **(born_opts or {}))
    elif gate == "sigmoid":
        step = lambda: cattn.pct_fwd(q, k, v, causal=w.causal, out=out)
    else:   # screening with r = 1, t = 0.5 (a threshold inside the score range)
        step = lambda: cattn.pct_gate_fwd(q, k, v, gate=gate, causal=w.causal, a=1.0, b=0.5, out=out)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    ev[0].record(stream)
    for i in range(steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t_wall) * 1e3
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    total_ms = ev[0].elapsed_time(ev[-1])
    return inp, from_device(out), total_ms / steps, per, wall_ms


def cpu_baseline(w, inp, got, budget_s: float = 12.0, gate: str = "sigmoid"):
    """The fp64 oracle on whole heads of the same inputs, as many heads as fit the budget.

    The heads it computes are also compared with the GPU output of the timed
    launches (row-wise relative error, the parity measure of the tests).
    """
    import oracle
    from threadpoolctl import threadpool_info
    from complex_valued_attention_amd.check import TOL, rowwise_rel_err
    from complex_valued_attention_amd.inputs import attention_flops

    if w.op == "born":
        fn = oracle.born_attention
    elif gate == "softmax":
        fn = oracle.pct_softmax_attention
    elif gate == "screen":   # the bench's screening parameters: r = 1, t = 0.5
        fn = lambda q, k, v, causal: oracle.pct_screen_attention(q, k, v, causal=causal, r=1.0, t=0.5)
    else:
        fn = oracle.pct_attention
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    done, t_used, err = 0, 0.0, 0.0
    for b, h in heads:
        t0 = time.perf_counter()
        ref = fn(inp.q64[b, h], inp.k64[b, h], inp.v64[b, h], causal=w.causal)
        t_used += time.perf_counter() - t0
        err = max(err, rowwise_rel_err(got[b, h], ref))
        done += 1
        if t_used >= budget_s:
            break
    flops = attention_flops(w.T, w.d_h, w.causal, done)
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {"value": flops / t_used / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} of {w.B * w.H} heads (full T={w.T} each), fp64 numpy, {t_used:.1f} s",
            **host_info(),
            "gpu_rowwise_rel_err": err, "gpu_parity_pass": bool(err <= TOL[w.layout])}


def host_info() -> dict:
    """nproc, the CPUs this process may run on, and the CPU model of the host."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return {"nproc": os.cpu_count(), "usable_cpus": usable, "cpu_model": model}


# The five workloads of the metric's config list, in its order: the headline is
# the fourth; the others are timed in the same run and reported beside it.
CONFIG_WORKLOADS = ["born_causal_c64_b1h1t128d16", "born_causal_c64_b4h8t1024d64_rotary",
                    "pct_full_c64_b8h8t2048d64", "born_causal_bf16_b8h16t4096d64_rotary",
                    "pct_causal_c64_b1h8t16384d64"]


def config_record(w, got, inp, ms, per, n_rows: int = 48) -> dict:
    """Timing, roofline fraction and sampled-row oracle parity of one workload."""
    import oracle
    from complex_valued_attention_amd import inputs as gen
    from complex_valued_attention_amd.check import TOL, rowwise_rel_err, sample_rows
    kernel_ms = float(np.mean(per))
    flops = gen.attention_flops(w.T, w.d_h, w.causal, w.B * w.H)
    alg = algorithmic_flops(w)
    peak = PEAK_TFLOPS[w.layout]
    rows = sample_rows(w.B, w.H, w.T, n_rows, seed=w.seed)
    fn = oracle.born_attention_rows if w.op == "born" else oracle.pct_attention_rows
    ref = fn(inp.q64, inp.k64, inp.v64, rows, causal=w.causal)
    err = rowwise_rel_err(got[rows[:, 0], rows[:, 1], rows[:, 2]], ref)
    achieved = alg / (kernel_ms * 1e-3) / 1e12
    # a single workgroup's worth of work cannot fill the chip: bound by launch latency
    latency = w.B * w.H * w.T <= 4096
    return {"op": w.op, "causal": w.causal, "B": w.B, "H": w.H, "T": w.T, "d_h": w.d_h, "layout": w.layout,
            "kernel": kernel_name(w), "kernel_ms_mean": kernel_ms, "kernel_ms_median": float(np.median(per)),
            "ms_per_step": ms,
            "flops_formula": flops, "flops_algorithmic": alg,
            "tflops_formula": flops / (kernel_ms * 1e-3) / 1e12, "tflops_algorithmic": achieved,
            "bound": "latency" if latency else "mfma", "peak_tflops": peak,
            "precision": "bf16 products, fp32 accumulation" if w.layout == "bf16" else "fp32",
            "frac": achieved / peak, "frac_of_bf16_peak": achieved / PEAK_TFLOPS["bf16"],
            "rows_checked": int(len(rows)), "rowwise_rel_err": err, "tol": TOL[w.layout],
            "parity_pass": bool(err <= TOL[w.layout])}


def option_records(w, inp, plain_ms: float, steps: int, warmup: int) -> dict:
    """The Born options on the headline workload, timed like it: the per-head
    decay (the fixed schedule of inputs.decay_gammas) and Q rotated at load
    (base 10000), each with sampled-row oracle parity."""
    import oracle
    from complex_valued_attention_amd import inputs as gen
    from complex_valued_attention_amd.check import TOL, rowwise_rel_err, sample_rows
    alg = algorithmic_flops(w)
    rows = sample_rows(w.B, w.H, w.T, 32, seed=w.seed)
    gam = gen.decay_gammas(w.H).astype(np.float32)
    out = {}
    for key, opts in (("decay", {"decay": gam}), ("rotary_q", {"rotary_base": 10000.0})):
        _, got, ms, per, _ = run_gpu(w, steps, warmup, born_opts=opts, inp=inp)
        if key == "decay":
            ref = oracle.born_attention_rows(inp.q64, inp.k64, inp.v64, rows, causal=w.causal,
                                             decay=gam.astype(np.float64))
        else:   # the oracle rotates the stored Q in fp64
            q64 = np.empty_like(inp.q64)
            for b in range(w.B):
                q64[b] = oracle.rotary(inp.q64[b], pos0=0, base=10000.0)
            ref = oracle.born_attention_rows(q64, inp.k64, inp.v64, rows, causal=w.causal)
            del q64
        err = rowwise_rel_err(got[rows[:, 0], rows[:, 1], rows[:, 2]], ref)
        kernel_ms = float(np.mean(per))
        achieved = alg / (kernel_ms * 1e-3) / 1e12
        out[key] = {"kernel": kernel_name(w), "kernel_ms_mean": kernel_ms, "kernel_ms_median": float(np.median(per)),
                    "tflops_algorithmic": achieved, "frac": achieved / PEAK_TFLOPS[w.layout],
                    "time_vs_plain": kernel_ms / plain_ms,
                    "rows_checked": int(len(rows)), "rowwise_rel_err": err, "tol": TOL[w.layout],
                    "parity_pass": bool(err <= TOL[w.layout])}
        if key == "decay":
            out[key]["gammas"] = "1 - 2^-(5 + 8 h / (H - 1)), h = 0..H-1 (0.969 .. 0.99988)"
        log(f"[bench] option {key}: {kernel_ms:.4f} ms ({kernel_ms / plain_ms:.3f} x plain), "
            f"frac {achieved / PEAK_TFLOPS[w.layout]:.3f}, parity {err:.2e}")
        del got
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="default run: skip timing the other four workloads beside the headline")
    ap.add_argument("--d-h", type=int, default=0,
                    help="--pass fwd/bwd: the named workload at this head width instead (not a headline number)")
    ap.add_argument("--pass", dest="which", choices=["fwd", "bwd", "rotary", "step", "linear"], default="fwd")
    ap.add_argument("--chunk", type=int, default=4096, help="--pass linear: tokens per chunk")
    ap.add_argument("--gate", choices=["sigmoid", "softmax", "screen"], default="sigmoid",
                    help="PCT workloads: the gate on the scaled cosine score")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="after the bench, run a plain elementwise copy of MIB MiB (reads and writes MIB MiB "
                         "per launch) five times: the reference kernel for scaling HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(heads shard across GPUs with no exchange; see the design notes). Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    from complex_valued_attention_amd import inputs as gen
    name = args.workload or gen.BENCH_WORKLOAD
    w = gen.WORKLOADS[name]
    if args.d_h:   # the named workload's shape and recipe at another head width
        name = f"{name}@d{args.d_h}"
        w = dataclasses.replace(w, d_h=args.d_h, name=name)

    if args.which == "bwd":
        main_bwd(args, w)
        if args.copy_probe:
            copy_probe(args.copy_probe)
        return
    if args.which == "rotary":
        main_rotary(args, w)
        if args.copy_probe:
            copy_probe(args.copy_probe)
        return
    if args.which == "step":
        main_step(args, w)
        if args.copy_probe:
            copy_probe(args.copy_probe)
        return
    if args.which == "linear":
        if args.workload is None:
            w = gen.WORKLOADS["born_causal_bf16_b1h16t32768d64_rotary"]
        main_linear(args, w)
        if args.copy_probe:
            copy_probe(args.copy_probe)
        return
    if args.gate != "sigmoid" and w.op != "pct":
        print("--gate applies to PCT workloads only", file=sys.stderr)
        sys.exit(2)
    inp, got, ms, per, wall_ms = run_gpu(w, args.steps, args.warmup, args.gate)
    flops = gen.attention_flops(w.T, w.d_h, w.causal, w.B * w.H)
    alg = algorithmic_flops(w)
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.layout]
    kernel_ms = float(np.mean(per))
    achieved = alg / (kernel_ms * 1e-3) / 1e12
    log(f"[bench] {name}: {ms:.4f} ms/step (median launch {np.median(per):.4f} ms, wall {wall_ms / args.steps:.4f} "
        f"ms/step), {tflops:.1f} TFLOP/s")

    rec = {
        "metric": METRIC if name == gen.BENCH_WORKLOAD else
        f"{w.op}{'' if args.gate == 'sigmoid' else '-' + args.gate} fwd real TFLOP/s ({name})",
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.layout == "bf16" else "f32",
        "data": "synthetic (seeded complex Gaussian, unit-norm rotary Q/K)" if w.rotary else "synthetic",
        "config": {"workload": name, "op": w.op, "causal": w.causal, "B": w.B, "H": w.H, "T": w.T,
                   "d_h": w.d_h, "layout": w.layout, "seed": w.seed,
                   **({} if args.gate == "sigmoid" else {"gate": args.gate})},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak,
                     "traffic": measured_traffic(name) if args.gate == "sigmoid" else None,
                     "kernel": kernel_name(w),
                     "kernel_ms_mean": kernel_ms, "kernel_ms_median": float(np.median(per))},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, inp, got, gate=args.gate)
        log(f"[bench] cpu baseline {rec['cpu_baseline']}")
    if args.workload is None and not args.d_h and not args.no_configs and w.op == "born":
        rec["options"] = option_records(w, inp, kernel_ms, args.steps, args.warmup)
    if args.workload is None and not args.d_h and not args.no_configs:
        # every workload of the metric's config list, timed in this run (the
        # headline's own entry repeats the numbers above)
        configs = {}
        for cname in CONFIG_WORKLOADS:
            if cname == name:
                configs[cname] = config_record(w, got, inp, ms, per)
                continue
            cw = gen.WORKLOADS[cname]
            cinp, cgot, cms, cper, _ = run_gpu(cw, args.steps, args.warmup)
            configs[cname] = config_record(cw, cgot, cinp, cms, cper)
            c = configs[cname]
            log(f"[bench] {cname}: {c['kernel_ms_mean']:.4f} ms, {c['tflops_algorithmic']:.1f} TFLOP/s "
                f"algorithmic, frac {c['frac']:.3f}, parity {c['rowwise_rel_err']:.2e}")
            del cinp, cgot
        rec["configs"] = configs
    print(json.dumps(rec), flush=True)
    if args.copy_probe:
        copy_probe(args.copy_probe)


def copy_probe(mib: int):
    """A kernel of known HBM traffic: y = -x over MIB MiB of fp32 (MIB MiB read, MIB MiB written)."""
    import torch
    n = mib * (1 << 20) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(5):
        torch.neg(x, out=y)
    torch.cuda.synchronize()
    log(f"[bench] copy probe: 5 launches of neg over {mib} MiB fp32 ({n * 4} bytes read and written each)")


if __name__ == "__main__":
    main()
