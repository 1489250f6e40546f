#!/usr/bin/env python3
"""Benchmark of the QLoRA NF4 + double-quant + LoRA linear on one MI355X.

One step = forward + backward (dX, dA, dB) of the three LLaMA-7B-shaped linears
4096->4096, 4096->11008, 11008->4096 at M = 4096 tokens, r = 64, alpha = 16, on
seeded synthetic bf16 inputs already resident in HBM.  The weights are quantized
(NF4 + 8-bit double quantization) once before timing; quantization throughput is
reported separately.  The headline value is algorithmic TFLOP/s,
4MNK + 6Mr(K+N) per linear (no dW is computed).

Also reported: the M = 1 forward weight stream (GB/s) on the 4096->11008 and
11008->4096 weights (r = 16, alpha = 32), replayed from a HIP graph over more than
512 MB of distinct weight copies so the bytes come from HBM; the roofline of the
dominant kernel (the fused NF4 GEMM, timed per launch with HIP events recorded by
the library on its launch stream, on every --time-every-th step of the timed region:
an event pair per launch costs a few microseconds of GPU time, so timing every launch
would slow the step it measures); and the CPU oracle timed on a bounded sample.

    python bench.py [--gpus 1] [--steps 20] [--warmup 15] [--time-every 4] [--no-cpu-baseline]
                    [--no-extras] [--m1-only [--small-m 1|4|16] | --merge-only | --calibrate-copy]
"""

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "NF4+LoRA linear fwd+bwd TFLOP/s at M=4096; weight-stream GB/s at M=1"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E


class HipEvents:
    """Raw hipEvent_t handles (the library records them on its launch stream)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.pool = []

    def pair(self):
        a, b = ctypes.c_void_p(), ctypes.c_void_p()
        if self.lib.hipEventCreate(ctypes.byref(a)) or self.lib.hipEventCreate(ctypes.byref(b)):
            raise RuntimeError("hipEventCreate failed")
        self.pool.append((a.value, b.value))
        return a.value, b.value

    def ms(self, a, b):
        out = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(out), a, b):
            raise RuntimeError("hipEventElapsedTime failed")
        return out.value

    def close(self):
        for a, b in self.pool:
            self.lib.hipEventDestroy(a)
            self.lib.hipEventDestroy(b)
        self.pool = []


def linear_flops(M, K, N, r):
    return 4 * M * N * K + 6 * M * r * (K + N)


def stream_bytes(M, K, N, r):
    n = N * K
    return n // 2 + n // 64 + 8 * ((n // 64 + 255) // 256) + 2 * r * (K + N) + 2 * M * K + 2 * M * N


def setup_workload2(torch, q, synth, gc):
    wl = synth.WORKLOADS[2]
    M = wl.M[0]
    L = []
    for i, (K, N) in enumerate(wl.linears):
        d = synth.workload_linear(2, i)
        W = gc.dev_weight(d)
        qw = q.quantize(W)
        e = dict(K=K, N=N, qw=qw, W=W, X=gc.dev_bf16(d["X"]), A=gc.dev_bf16(d["A"]),
                 B=gc.dev_bf16(d["B"]), dY=gc.dev_bf16(d["dY"]))
        e["Y"] = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        e["U"] = torch.empty((M, wl.r), dtype=torch.bfloat16, device="cuda")
        e["dX"] = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
        e["dA"] = torch.empty((wl.r, K), dtype=torch.bfloat16, device="cuda")
        e["dB"] = torch.empty((N, wl.r), dtype=torch.bfloat16, device="cuda")
        e["ws"] = q.workspace(1, M, K, N, wl.r, "cuda")
        e["wsf"] = q.workspace(0, M, K, N, wl.r, "cuda")
        L.append(e)
    return wl, M, L


def run_step(q, wl, L, ev=None, record=None):
    for e in L:
        if ev is not None:
            a, b = ev.pair()
            q._lib.qlora_time_next_gemm(a, b)
            record.append((a, b, "fwd", e))
        q.linear_fwd(e["qw"], e["X"], e["A"], e["B"], wl.alpha, Y=e["Y"], U=e["U"], ws=e["wsf"])
        if ev is not None:
            a, b = ev.pair()
            q._lib.qlora_time_next_gemm(a, b)
            record.append((a, b, "dx", e))
        q.linear_bwd(e["qw"], e["dY"], e["X"], e["A"], e["B"], wl.alpha, e["U"], dX=e["dX"],
                     dA=e["dA"], dB=e["dB"], ws=e["ws"])


def measure_quantize(torch, q, L, reps=5):
    """Quantization of each workload-2 weight, `reps` calls replayed from a HIP graph: a
    call on these sizes runs 14-28 us on the GPU, about what the binding takes on the host
    (four output allocations and the ctypes call), so eager back-to-back calls would time
    the host."""
    t = []
    elems = 0
    for e in L:
        for _ in range(2):
            q.quantize(e["W"])
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                q.quantize(e["W"])
        g.replay()
        torch.cuda.synchronize()
        s, f = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        g.replay()
        f.record()
        torch.cuda.synchronize()
        t.append(s.elapsed_time(f) / reps)
        elems += e["K"] * e["N"]
        del g
    ms = sum(t)
    return {"value": round(elems * 2.516 / (ms * 1e-3) / 1e9, 1), "unit": "GB/s",
            "bytes_per_weight": 2.516, "ms_three_weights": round(ms, 4),
            "frac_of_hbm_peak": round(elems * 2.516 / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "what": "bf16 -> NF4 codes + int8 DQ constants, the three workload-2 weights (HIP-graph replay)"}


def measure_quantize_stress(torch, q, synth, gc, copies=12, reps=2):
    """Quantization stress workload: NF4 + int8 DQ over a stream of 8192 x 22016 bf16 weights
    (Student-t(3) x 0.02 with 0.1 % outliers at +-50 std and one zero block per row): `copies`
    distinct seeded matrices drawn on the device (about 4.3 GB of bf16 at 12), so every
    quantization streams a different weight from HBM."""
    from synth.device import stress_weight_device
    wl = synth.WORKLOADS[5]
    K, N = wl.linears[0]
    Ws = [stress_weight_device([5, i], N, K) for i in range(copies)]
    W0 = Ws[0]
    for W in Ws[:2]:  # outputs come from torch's caching allocator: no allocation in the timed loop
        q.quantize(W)
    torch.cuda.synchronize()
    s, f = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        for W in Ws:
            q.quantize(W)
    f.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(f) / (reps * copies)
    gbs = N * K * 2.516 / (ms * 1e-3) / 1e9
    quant = {"value": round(gbs, 1), "unit": "GB/s", "bytes_per_weight": 2.516, "ms_per_weight": round(ms, 4),
             "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4), "stream_GB": round(copies * N * K * 2 / 1e9, 2),
             "what": f"bf16 -> NF4 codes + int8 DQ constants, {N}x{K} stress weights (Student-t(3), outliers, "
                     f"zero blocks), {copies} distinct seeded matrices"}
    # standalone decode of the same stream: the quantized copies -> one bf16 output buffer
    qws = [q.quantize(W) for W in Ws]
    quant["error"] = stress_error(torch, q, W0, qws[0])
    del Ws, W0
    out = torch.empty((N, K), dtype=torch.bfloat16, device="cuda")
    q.dequantize(qws[0], out=out)
    torch.cuda.synchronize()
    s.record()
    for _ in range(reps):
        for qw in qws:
            q.dequantize(qw, out=out)
    f.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(f) / (reps * copies)
    gbs = N * K * 2.516 / (ms * 1e-3) / 1e9
    deq = {"value": round(gbs, 1), "unit": "GB/s", "bytes_per_weight": 2.516, "ms_per_weight": round(ms, 4),
           "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
           "what": f"NF4 codes + int8 DQ constants -> bf16 (standalone doubleDequant), the {copies} quantized "
                   f"{N}x{K} stress weights"}
    del qws, out
    return quant, deq


def stress_error(torch, q, W, qw, outlier_abs=0.5):
    """Decode error of one stress weight, from the library's own dequantize: per 64-block
    absmax c of W, the max and RMS of |w - w'| / c over three kinds of blocks (all-zero,
    blocks holding an outlier |w| >= outlier_abs, the rest), and the max absolute error in
    the zero blocks (it must be 0)."""
    Wd = q.dequantize(qw).float().view(-1, 64)
    Wf = W.float().view(-1, 64)
    c = Wf.abs().amax(dim=1)
    err = (Wf - Wd).abs()
    zero = c == 0
    outl = (~zero) & (Wf.abs() >= outlier_abs).any(dim=1)
    bulk = (~zero) & (~outl)
    out = {"blocks": int(c.numel()), "zero_blocks": int(zero.sum()), "outlier_blocks": int(outl.sum()),
           "max_abs_err_zero_blocks": float(err[zero].max()) if bool(zero.any()) else 0.0}
    for name, sel in (("bulk", bulk), ("outlier", outl)):
        if bool(sel.any()):
            rel = err[sel] / c[sel].unsqueeze(1)
            out[name] = {"max_err_over_c": round(float(rel.max()), 6),
                         "rms_err_over_c": round(float(rel.pow(2).mean().sqrt()), 6)}
    out["what"] = ("|w - w'| / c per 64-block (c = block absmax), first stress matrix: NF4's half-gap between "
                   "adjacent levels (at most 0.16) plus |q| |c - c'| / c from the int8 double quantization of c, "
                   "which is large for blocks of small c in groups of 256 blocks that also hold outlier blocks")
    return out


def step_percentiles(ms):
    v = sorted(ms)
    pick = lambda f: v[min(len(v) - 1, max(0, int(round(f * (len(v) - 1)))))]  # noqa: E731
    return {"p10": round(pick(0.1), 4), "p50": round(pick(0.5), 4), "p90": round(pick(0.9), 4),
            "min": round(v[0], 4), "max": round(v[-1], 4), "n": len(v)}


def measure_config1(torch, q, synth, gc, calls=200):
    """Workload 1 (one 1024 -> 1024 linear, M = 64, r = 8, W drawn fp32): device time of one
    forward + backward (dX, dA, dB), replayed from a HIP graph, with B = 0 and with
    B ~ N(0, 0.01^2)."""
    wl = synth.WORKLOADS[1]
    K, N = wl.linears[0]
    M = wl.M[0]
    d = synth.workload_linear(1, 0)
    qw = q.quantize(gc.dev_weight(d))
    X, A, Bn, dY = gc.dev_bf16(d["X"]), gc.dev_bf16(d["A"]), gc.dev_bf16(d["B"]), gc.dev_bf16(d["dY"])
    out = {"what": "1024->1024, M=64, r=8, alpha=16: one forward + backward per call, graph-replayed"}
    for name, B in (("B_zero", torch.zeros_like(Bn)), ("B_normal", Bn)):
        Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        U = torch.empty((M, wl.r), dtype=torch.bfloat16, device="cuda")
        dX = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
        dA = torch.empty((wl.r, K), dtype=torch.bfloat16, device="cuda")
        dB = torch.empty((N, wl.r), dtype=torch.bfloat16, device="cuda")
        wsf, wsb = q.workspace(0, M, K, N, wl.r, "cuda"), q.workspace(1, M, K, N, wl.r, "cuda")

        def one():
            q.linear_fwd(qw, X, A, B, wl.alpha, Y=Y, U=U, ws=wsf)
            q.linear_bwd(qw, dY, X, A, B, wl.alpha, U, dX=dX, dA=dA, dB=dB, ws=wsb)
        one()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(calls):
                one()
        g.replay()
        torch.cuda.synchronize()
        s, f = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(3):
            g.replay()
        f.record()
        torch.cuda.synchronize()
        us = s.elapsed_time(f) * 1e3 / (3 * calls)
        out[name] = {"us_per_fwd_bwd": round(us, 2),
                     "TFLOP/s": round(linear_flops(M, K, N, wl.r) / (us * 1e-6) / 1e12, 3)}
    return out


def measure_ceilings(torch, M=4096, shapes=((4096, 4096), (4096, 11008), (11008, 4096)), reps=10):
    """Practical ceilings on this GPU: a plain device copy (read + write bytes per second) and
    torch's bf16 GEMM (hipBLASLt) on the workload's dense shapes X [M, K] . W^T [K, N]."""
    n = 512 << 20  # bf16 elements (1 GiB)
    src = torch.empty(n, dtype=torch.bfloat16, device="cuda").normal_()
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    s, f = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        dst.copy_(src)
    f.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(f) / reps
    out = {"copy_GB/s": round(4 * n / (ms * 1e-3) / 1e9, 1),
           "copy_what": "1 GiB bf16 device copy, read + write bytes"}
    del src, dst
    mm = {}
    for K, N in shapes:
        X = torch.randn(M, K, device="cuda").to(torch.bfloat16)
        Wt = torch.randn(K, N, device="cuda").to(torch.bfloat16).contiguous()
        torch.matmul(X, Wt)
        torch.cuda.synchronize()
        s.record()
        for _ in range(reps):
            torch.matmul(X, Wt)
        f.record()
        torch.cuda.synchronize()
        ms = s.elapsed_time(f) / reps
        mm[f"{K}->{N}"] = {"us": round(ms * 1e3, 1), "TFLOP/s": round(2 * M * N * K / (ms * 1e-3) / 1e12, 1)}
        del X, Wt
    out["torch_matmul_bf16_M4096"] = mm
    return out


def environment(torch):
    props = torch.cuda.get_device_properties(0)
    rocm = None
    try:
        rocm = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        pass
    return {"gpu": torch.cuda.get_device_name(0), "compute_units": props.multi_processor_count,
            "hbm_GB": round(props.total_memory / 1e9, 1), "gcn_arch": getattr(props, "gcnArchName", None),
            "rocm": rocm, "torch": torch.__version__, "hip": torch.version.hip,
            "python": sys.version.split()[0], "host_cores": os.cpu_count(),
            "seeds": "synth: numpy default_rng([workload - 1, linear, M]) per linear, drawing W, X, A, B, dY "
                     "in that order; stress matrices: torch.Generator seeded from [5, i]"}


def measure_m1(torch, q, synth, gc, ev, M=1, min_bytes=600 << 20, calls=200):
    """Small-M forward (M = 1, 4 or 16) over distinct weight copies, replayed from a HIP graph."""
    wl = synth.WORKLOADS[3]
    out = {"M": M, "per_linear": []}
    tot_bytes = tot_ms = 0.0
    for i, (K, N) in enumerate(wl.linears):
        d = synth.workload_linear(3, i, M=M, parts=("W", "X", "A", "B"))
        qw0 = q.quantize(gc.dev_weight(d))
        wbytes = qw0.codes.numel() + qw0.absmax_q.numel() + 8 * qw0.dq_scale.numel()
        copies = max(2, -(-min_bytes // wbytes))
        qws = [q.NF4Weight(qw0.codes.clone(), qw0.absmax_q.clone(), qw0.dq_scale.clone(),
                           qw0.dq_offset.clone(), qw0.n_rows, qw0.n_cols) for _ in range(copies)]
        X, A, B = gc.dev_bf16(d["X"]), gc.dev_bf16(d["A"]), gc.dev_bf16(d["B"])
        Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        U = torch.empty((M, wl.r), dtype=torch.bfloat16, device="cuda")
        wsf = q.workspace(0, M, K, N, wl.r, "cuda")
        for c in range(copies):  # warm up, and make sure every copy works eagerly
            q.linear_fwd(qws[c], X, A, B, wl.alpha, Y=Y, U=U, ws=wsf)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for c in range(calls):
                q.linear_fwd(qws[c % copies], X, A, B, wl.alpha, Y=Y, U=U, ws=wsf)
        g.replay()
        torch.cuda.synchronize()
        s, f = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        reps = 5
        for _ in range(reps):
            g.replay()
        f.record()
        torch.cuda.synchronize()
        ms_call = s.elapsed_time(f) / (reps * calls)
        # kernel-only time of the GEMV (event hook, eager launches)
        rec = []
        for c in range(copies):
            a, b = ev.pair()
            q._lib.qlora_time_next_gemm(a, b)
            q.linear_fwd(qws[c], X, A, B, wl.alpha, Y=Y, U=U, ws=wsf)
        torch.cuda.synchronize()
        kms = sum(ev.ms(a, b) for a, b in ev.pool[-copies:]) / copies
        nb = stream_bytes(M, K, N, wl.r)
        out["per_linear"].append({"K": K, "N": N, "us_per_call": round(ms_call * 1e3, 3),
                                  "GB/s": round(nb / (ms_call * 1e-3) / 1e9, 1),
                                  "gemv_kernel_us": round(kms * 1e3, 3),
                                  "gemv_kernel_GB/s": round(nb / (kms * 1e-3) / 1e9, 1),
                                  "weight_copies": copies})
        tot_bytes += nb
        tot_ms += ms_call
        del qws
    out.update({"value": round(tot_bytes / (tot_ms * 1e-3) / 1e9, 1), "unit": "GB/s",
                "frac_of_hbm_peak": round(tot_bytes / (tot_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                "bytes_per_call": "N*K/2 + N*K/64 + 8*groups + 2r(K+N) + 2MK + 2MN",
                "timing": "HIP graph replay of 200 calls over >512 MB of weight copies"})
    return out


def weight_bytes(qw):
    """Stored bytes of a quantized weight (codes and block / group constants)."""
    return sum(a.numel() * a.element_size() for a in (qw.codes, qw.absmax_q, qw.dq_scale, qw.dq_offset,
                                                      qw.absmax) if a is not None)


def measure_variants(torch, q, synth, gc, wl, L, ev, steps=10, warmup=10, min_bytes=600 << 20, calls=20):
    """The data-type variants (level table x block-constant type) on the same work: the
    M = 4096 training step of the three workload-2 linears, and the M = 1 forward
    kernel on the 4096 -> 11008 weight streamed over distinct copies (bytes as stored)."""
    import dataclasses
    out = {}
    names = {(0, 0): "nf4+dq_int8", (0, 1): "nf4+dq_fp8", (0, 2): "nf4+fp32",
             (1, 0): "fp4+dq_int8", (1, 1): "fp4+dq_fp8", (1, 2): "fp4+fp32"}
    M = L[0]["X"].shape[0]
    flops = sum(linear_flops(M, e["K"], e["N"], wl.r) for e in L)
    d1 = synth.workload_linear(3, 0, M=1, parts=("W", "X", "A", "B"))
    w1 = gc.dev_weight(d1)
    X1, A1, B1 = gc.dev_bf16(d1["X"]), gc.dev_bf16(d1["A"]), gc.dev_bf16(d1["B"])
    r1, alpha1 = A1.shape[0], synth.WORKLOADS[3].alpha
    K1, N1 = w1.shape[1], w1.shape[0]
    Y1 = torch.empty((1, N1), dtype=torch.bfloat16, device="cuda")
    ws1 = q.workspace(0, 1, K1, N1, r1, "cuda")
    for (qt, ct), name in names.items():
        Lv = [dict(e, qw=q.quantize(e["W"], quant_type=qt, const_type=ct)) for e in L]
        for _ in range(warmup):
            run_step(q, wl, Lv)
        torch.cuda.synchronize()
        s, f = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(steps):
            run_step(q, wl, Lv)
        f.record()
        torch.cuda.synchronize()
        ms = s.elapsed_time(f) / steps
        del Lv
        qw0 = q.quantize(w1, quant_type=qt, const_type=ct)
        wb = weight_bytes(qw0)
        copies = max(2, -(-min_bytes // wb))
        qws = [dataclasses.replace(qw0, **{k: (getattr(qw0, k).clone() if getattr(qw0, k) is not None else None)
                                           for k in ("codes", "absmax_q", "dq_scale", "dq_offset", "absmax")})
               for _ in range(copies)]
        for c in range(copies):
            q.linear_fwd(qws[c], X1, A1, B1, alpha1, Y=Y1, save_u=False, ws=ws1)
        torch.cuda.synchronize()
        n0 = len(ev.pool)
        for i in range(calls):
            a, b = ev.pair()
            q._lib.qlora_time_next_gemm(a, b)
            q.linear_fwd(qws[i % copies], X1, A1, B1, alpha1, Y=Y1, save_u=False, ws=ws1)
        torch.cuda.synchronize()
        kms = sum(ev.ms(a, b) for a, b in ev.pool[n0:]) / calls
        nb = wb + 2 * r1 * (K1 + N1) + 2 * K1 + 2 * N1
        out[name] = {"step_ms": round(ms, 4), "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 1),
                     "m1_kernel_us": round(kms * 1e3, 2), "m1_kernel_GB/s": round(nb / (kms * 1e-3) / 1e9, 1),
                     "weight_bytes": wb}
        del qws
    ev.close()
    out["what"] = ("per variant: fwd+bwd step of the three workload-2 linears at M=4096 (TFLOP/s as the "
                   "headline); M=1 GEMV kernel on 4096->11008 over >512 MB of weight copies (GB/s of "
                   "the bytes the variant stores, plus adapter, X and Y)")
    return out


def measure_adamw(torch, q, reps=20):
    """AdamW step over the adapters of the LLaMA-65B layer (r = 64 on all seven linears):
    fp32 parameter and moments, bf16 gradient, bf16 parameter copy; 28 bytes per value."""
    n = 4 * 64 * (8192 + 8192) + 2 * 64 * (8192 + 22016) + 64 * (22016 + 8192)
    g = torch.Generator(device="cuda").manual_seed(4)
    p = torch.randn(n, device="cuda", generator=g) * 0.02
    grad = (torch.randn(n, device="cuda", generator=g) * 0.05).to(torch.bfloat16)
    m = torch.zeros_like(p)
    v = torch.zeros_like(p)
    pb = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    for t in range(1, 4):
        q.adamw_step(p, grad, m, v, t, 2e-4, weight_decay=0.01, param_bf16=pb)
    torch.cuda.synchronize()
    s, f = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for t in range(4, 4 + reps):
        q.adamw_step(p, grad, m, v, t, 2e-4, weight_decay=0.01, param_bf16=pb)
    f.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(f) / reps
    gbs = 28 * n / (ms * 1e-3) / 1e9
    return {"value": round(gbs, 1), "unit": "GB/s", "us_per_step": round(ms * 1e3, 2), "params": n,
            "bytes_per_param": 28, "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
            "what": "AdamW step on the 65B layer's LoRA adapters (fp32 state, bf16 grad and copy)"}


def measure_merge(torch, q, reps=10):
    """LoRA merge into bf16 (and unmerge) on the 65B layer's 8192 -> 22016 weight, r = 64:
    algorithmic HBM bytes 0.516 + 2 per weight (merge), 2 + 2 (unmerge)."""
    N, K, r = 22016, 8192, 64
    g = torch.Generator(device="cuda").manual_seed(5)
    W = (torch.randn(N, K, device="cuda", generator=g) * 0.015).to(torch.bfloat16)
    qw = q.quantize(W)
    del W
    A = (torch.randn(r, K, device="cuda", generator=g) * (1.0 / r) ** 0.5).to(torch.bfloat16)
    B = (torch.randn(N, r, device="cuda", generator=g) * 0.01).to(torch.bfloat16)
    out = torch.empty(N, K, dtype=torch.bfloat16, device="cuda")
    back = torch.empty_like(out)
    res = {}
    for name, fn, bpw in (("merge", lambda: q.lora_merge(qw, A, B, 16.0, out=out), 0.5 + 1 / 64 + 2),
                          ("unmerge", lambda: q.lora_unmerge(out, A, B, 16.0, out=back), 4.0)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        s, f = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            fn()
        f.record()
        torch.cuda.synchronize()
        ms = s.elapsed_time(f) / reps
        gbs = bpw * N * K / (ms * 1e-3) / 1e9
        res[name] = {"value": round(gbs, 1), "unit": "GB/s", "us": round(ms * 1e3, 2),
                     "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}
    res["what"] = "LoRA merge / unmerge, 22016 x 8192 bf16 output, r = 64"
    return res


def measure_layer65b(torch, q, reps=5, warmup=4):
    """LLaMA-65B decoder layer (M = 2048, r = 64, all seven linears, fwd + bwd): the
    linears one by one, and with q/k/v and gate/up horizontally fused (one weight stream
    and one GEMM each for the shared X)."""
    M, r, alpha, D, F = 2048, 64, 16.0, 8192, 22016
    g = torch.Generator(device="cuda").manual_seed(6)

    def weight(N, K):
        W = (torch.randn(N, K, device="cuda", generator=g) * 0.015).to(torch.bfloat16)
        qw = q.quantize(W)
        del W
        return qw

    def bf(*shape, std=1.0):
        return (torch.randn(*shape, device="cuda", generator=g) * std).to(torch.bfloat16)

    names = ("q", "k", "v", "o", "gate", "up", "down")
    shapes = {"q": (D, D), "k": (D, D), "v": (D, D), "o": (D, D), "gate": (F, D), "up": (F, D),
              "down": (D, F)}  # (N, K)
    qw = {n: weight(*shapes[n]) for n in names}
    A = {n: bf(r, shapes[n][1], std=(1.0 / r) ** 0.5) for n in names}
    B = {n: bf(shapes[n][0], r, std=0.01) for n in names}
    X = bf(M, D)
    Xd = bf(M, F)  # the down projection's input
    dY = {n: bf(M, shapes[n][0]) for n in names}
    flops = sum(linear_flops(M, shapes[n][1], shapes[n][0], r) for n in names)

    def separate():
        for n in names:
            x = Xd if n == "down" else X
            Y, U = q.linear_fwd(qw[n], x, A[n], B[n], alpha)
            q.linear_bwd(qw[n], dY[n], x, A[n], B[n], alpha, U)

    fq = q.concat_rows([qw["q"], qw["k"], qw["v"]])
    fg = q.concat_rows([qw["gate"], qw["up"]])
    Aq, Bq = torch.cat([A["q"], A["k"], A["v"]]), torch.cat([B["q"], B["k"], B["v"]])
    Ag, Bg = torch.cat([A["gate"], A["up"]]), torch.cat([B["gate"], B["up"]])
    dYq = torch.cat([dY["q"], dY["k"], dY["v"]], dim=1)
    dYg = torch.cat([dY["gate"], dY["up"]], dim=1)

    def fused():
        Y, U = q.linear_fwd_fused(fq, 3, X, Aq, Bq, alpha)
        q.linear_bwd_fused(fq, 3, dYq, X, Aq, Bq, alpha, U)
        Y, U = q.linear_fwd(qw["o"], X, A["o"], B["o"], alpha)
        q.linear_bwd(qw["o"], dY["o"], X, A["o"], B["o"], alpha, U)
        Y, U = q.linear_fwd_fused(fg, 2, X, Ag, Bg, alpha)
        q.linear_bwd_fused(fg, 2, dYg, X, Ag, Bg, alpha, U)
        Y, U = q.linear_fwd(qw["down"], Xd, A["down"], B["down"], alpha)
        q.linear_bwd(qw["down"], dY["down"], Xd, A["down"], B["down"], alpha, U)

    res = {}
    for name, fn in (("separate", separate), ("fused", fused)):
        # the step time settles over a few tens of milliseconds of work after an idle gap
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        s, f = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            fn()
        f.record()
        torch.cuda.synchronize()
        ms = s.elapsed_time(f) / reps
        res[name] = {"ms": round(ms, 3), "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 1)}
    res["speedup"] = round(res["separate"]["ms"] / res["fused"]["ms"], 3)
    res["what"] = ("LLaMA-65B layer, M=2048, r=64, 7 linears fwd+bwd; fused = q/k/v and gate/up as "
                   "one weight each (qlora_linear_*_fused)")
    res["flops_per_layer"] = flops
    return res


def cpu_baseline(synth, sample_m=4096, min_seconds=10.0, max_passes=20):
    """The oracle (float64 numpy) on a bounded sample of the workload: the three linears
    with the first `sample_m` tokens (decode of W' from the stored format, forward and
    backward), repeated until at least `min_seconds` of CPU work.  The oracle's own
    quantization of W is done once, untimed."""
    import numpy as np
    from oracle import linear, nf4
    wl = synth.WORKLOADS[2]
    cases = []
    tq = nq = 0.0
    for i, (K, N) in enumerate(wl.linears):
        d = synth.workload_linear(2, i)
        Wf = synth.bf16_bits_to_f32(d["W"])
        t0 = time.perf_counter()
        qw = nf4.quantize_nf4(Wf)
        tq += time.perf_counter() - t0
        nq += Wf.size
        f = lambda k: synth.bf16_bits_to_f32(d[k]).astype(np.float64)  # noqa: E731
        cases.append((K, N, qw, f("X")[:sample_m], f("A"), f("B"), f("dY")[:sample_m]))
        del d, Wf
    dt = fl = 0.0
    per = {"dequantize": 0.0, "forward": 0.0, "backward": 0.0}
    passes = 0
    while passes < max_passes and (passes == 0 or dt < min_seconds):
        for K, N, qw, X, A, B, dY in cases:
            t0 = time.perf_counter()
            Wd = nf4.dequantize_bf16(qw)
            t1 = time.perf_counter()
            linear.forward(X, Wd, A, B, wl.alpha, wl.r)
            t2 = time.perf_counter()
            linear.backward(dY, X, Wd, A, B, wl.alpha, wl.r)
            t3 = time.perf_counter()
            per["dequantize"] += t1 - t0
            per["forward"] += t2 - t1
            per["backward"] += t3 - t2
            dt += t3 - t0
            fl += linear_flops(sample_m, K, N, wl.r)
        passes += 1
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count()
    return {"value": round(fl / dt / 1e12, 4), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "seconds": round(dt, 2), "passes": passes,
            "per_step_ms": {k: round(v * 1e3 / passes, 1) for k, v in per.items()},
            "quantize": {"seconds": round(tq, 2), "weights": int(nq),
                         "Mweights_per_s": round(nq / tq / 1e6, 3) if tq > 0 else None,
                         "what": "the oracle's NF4 + double quantization of the three weights, once"},
            "sample": f"the three linears of the workload with the first {sample_m} of 4096 tokens, "
                      f"{passes} passes: decode W' + forward + backward in float64 numpy "
                      "(quantization untimed)"}


GEMM_SOURCES = ("bit_quantized_lora_nf4_amd/csrc/gemm.hip", "bit_quantized_lora_nf4_amd/csrc/device_common.h")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_nf4_workload2_traffic.md")


def gemm_source_hash():
    import hashlib
    h = hashlib.sha256()
    for rel in GEMM_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic():
    """HBM bytes per fused-GEMM launch from the committed counter summary, or None when
    the kernels have changed since the counters were taken."""
    try:
        lines = open(TRAFFIC_FILE).read().splitlines()
    except OSError:
        return None
    kv = {}
    for line in lines:
        if line.startswith("- ") and ": " in line:
            k, v = line[2:].split(": ", 1)
            kv[k.strip()] = v.strip().strip("`")
    if kv.get("gemm_source_sha256_16") != gemm_source_hash():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def calibrate_copy(torch, mib=1024, reps=5):
    """A plain device copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    n = mib * (1 << 20) // 2
    src = torch.randn(n, device="cuda").to(torch.bfloat16)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n * 2, "copy_bytes_written": n * 2, "reps": reps}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=15)
    ap.add_argument("--time-every", type=int, default=4,
                    help="record the GEMM launch events on every n-th timed step (1 = every step)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the M=1 and quantize legs")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 1 GiB device copy (counter calibration) and exit")
    ap.add_argument("--m1-only", action="store_true",
                    help="only run the M=1 weight-stream leg (for profiling the small-M forward) and exit")
    ap.add_argument("--small-m", type=int, default=1, choices=(1, 4, 16),
                    help="token count of the --m1-only leg (default 1)")
    ap.add_argument("--merge-only", action="store_true",
                    help="only run the LoRA merge / unmerge leg (for profiling it) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build measures one GPU only; --gpus must be 1 "
              "(the data-parallel all-reduce of dA/dB is not built).", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.calibrate_copy:
        calibrate_copy(torch)
        return
    import bit_quantized_lora_nf4_amd as q
    import synth
    from synth import device as gc
    if args.merge_only:
        print(json.dumps({"lora_merge": measure_merge(torch, q)}), flush=True)
        return
    if args.m1_only:
        ev = HipEvents()
        key = "weight_stream_m%d" % args.small_m
        print(json.dumps({key: measure_m1(torch, q, synth, gc, ev, M=args.small_m)}), flush=True)
        ev.close()
        return

    print("bench: setting up workload 2 (3 linears, M=4096)", file=sys.stderr, flush=True)
    wl, M, L = setup_workload2(torch, q, synth, gc)
    ev = HipEvents()
    for _ in range(args.warmup):
        run_step(q, wl, L)
    torch.cuda.synchronize()
    rec = []
    t0 = time.perf_counter()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    marks[0].record()
    every = max(1, args.time_every)
    for i in range(args.steps):
        if i % every == 0:
            run_step(q, wl, L, ev, rec)
        else:
            run_step(q, wl, L)
        marks[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = marks[0].elapsed_time(marks[-1]) / args.steps
    step_ms = [marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps)]
    flops_step = sum(linear_flops(M, e["K"], e["N"], wl.r) for e in L)
    value = flops_step / (ms_step * 1e-3) / 1e12
    print(f"bench: {args.steps} steps, {ms_step:.3f} ms/step (wall {wall:.2f} s)", file=sys.stderr,
          flush=True)

    g_fl = g_ms = 0.0
    per = {}
    for a, b, kind, e in rec:
        ms = ev.ms(a, b)
        fl = 2 * M * e["N"] * e["K"] + 2 * M * wl.r * (e["N"] if kind == "fwd" else e["K"])
        g_fl += fl
        g_ms += ms
        key = f"{kind} {e['K']}->{e['N']}"
        per.setdefault(key, [0.0, 0.0, 0])
        per[key][0] += fl
        per[key][1] += ms
        per[key][2] += 1
    achieved = g_fl / (g_ms * 1e-3) / 1e12
    roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": recorded_traffic(),
            "traffic_unit": "HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "kernel": "fused NF4-decode GEMM (forward and dX launches; a dX launch also carries dA's finalize pass)",
            "per_launch_flops": "fwd 2MNK + 2MNr; dX 2MNK + 2MKr",
            "avg_launch_us": round(g_ms * 1e3 / max(1, len(rec)), 2),
            "per_shape": {k: {"TFLOP/s": round(v[0] / (v[1] * 1e-3) / 1e12, 1),
                              "avg_us": round(v[1] * 1e3 / v[2], 1)} for k, v in per.items()},
            "timed_launches": len(rec),
            "timed_steps": f"one step in {every} of the {args.steps} timed steps",
            "step_time_in_gemm": round(g_ms / len(range(0, args.steps, every)) / ms_step, 4)}

    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,.02^2) bf16 weights NF4+DQ-quantized; X, dY ~ N(0,1))",
        "config": {"workload": "LLaMA-7B linears 4096->4096, 4096->11008, 11008->4096; fwd+bwd",
                   "M": M, "r": wl.r, "alpha": wl.alpha, "block": 64, "dq_group": 256,
                   "parallelism": "single GPU"},
        "roofline": roof,
        "step_ms": dict(step_percentiles(step_ms),
                        note="per-step durations of the timed steps (steps with GEMM event timing included)"),
        "environment": environment(torch),
    }
    ev.close()
    if not args.no_extras:
        print("bench: workload 1 latency and ceilings", file=sys.stderr, flush=True)
        result["config1_latency"] = measure_config1(torch, q, synth, gc)
        result["ceilings"] = measure_ceilings(torch)
        print("bench: M=1 weight stream", file=sys.stderr, flush=True)
        result["weight_stream_m1"] = measure_m1(torch, q, synth, gc, ev)
        ev.close()
        for m in (4, 16):
            result[f"weight_stream_m{m}"] = measure_m1(torch, q, synth, gc, ev, M=m)
            ev.close()
        result["quantize"] = measure_quantize(torch, q, L)
        print("bench: quantization stress stream", file=sys.stderr, flush=True)
        result["quantize_stress"], result["dequantize_stress"] = measure_quantize_stress(torch, q, synth, gc)
        result["adamw"] = measure_adamw(torch, q)
        result["lora_merge"] = measure_merge(torch, q)
        result["layer65b"] = measure_layer65b(torch, q)
        print("bench: data-type variants", file=sys.stderr, flush=True)
        result["variants"] = measure_variants(torch, q, synth, gc, wl, L, ev)
    if not args.no_cpu_baseline:
        print("bench: CPU oracle baseline", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(synth)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
