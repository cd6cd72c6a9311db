#!/usr/bin/env python3
"""Throughput of SignRot's fused online path on one MI355X.

One step = one call of signrot_rotate_quant_int4_outlier (the online path
with the calibrated sign vector d = sigma * row c of H, passed as (c, sigma))
over a whole batch: bf16
activations in HBM -> Hadamard rotation -> sign flip -> per-token min/max ->
scale, zero-point -> rounding -> packed int4 codes in HBM.  Calibration is an
offline step and is not timed.

Workload: n = 14336 (= 28 * 2^9, the LLaMA3-8B down-projection input width),
8192 tokens per batch, background N(0, 0.7) with a massive outlier channel
(M ~ U[800, 2500]) in 20% of tokens, seeded and synthetic.

The inputs are copied to several device buffers whose total exceeds the
256 MiB last-level (MALL) cache, and the steps cycle through them, so every
step reads its input from HBM.

Before the headline steps, three auxiliary legs run on the same buffers, each
with its own warm-up: a traffic-ceiling kernel that moves the same bytes per
token with no arithmetic, the d-vector entry point signrot_rotate_quant_int4,
and the integer zero-point variant.  The line also reports per-launch
percentiles, the quantization MSE of the GPU's own outputs, and the
decode-sized latency.

With the default workload the line also times the other configurations
(n = 4096 x 64, 8192 x 2048, 14336 x 4096, 28672 x 8192 tokens) after the
headline, each beside the traffic-ceiling kernel on the same buffers.

Prints one JSON line.  Flags: --gpus N (only 1 is supported), --steps K,
--warmup W, --workload W, --no-cpu-baseline, --no-decode (skip the
decode-latency leg and the other configurations, so that only the named
workload's kernels run), --pmc-copy (also run plain copies of known size for the
counter calibration of a rocprofv3 --pmc run); --fold times the offline weight
fold, --linear the INT4-activation down-projection and --swiglu the path with
the SwiGLU producer fused in, instead.
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

PEAK_HBM_GBS = 8000.0  # MI355X published HBM3E bandwidth
WORKLOAD = "n14336_t8192"
BUFFER_SETS_MIN_BYTES = 1.2 * 2**30
# Sources that define the timed kernel; the HBM traffic measured with
# rocprofv3 counters is reported only while they are unchanged.
# (plus the compile flags, build.COMMON)
_CSRC = "rotation_activation_quantization_amd/csrc/"
KERNEL_SOURCES = (_CSRC + "rq_fast.hip", _CSRC + "rq_fast_common.h", _CSRC + "wave_ops.h", _CSRC + "device_common.h",
                  _CSRC + "internal.h")
HALVES_SOURCES = (_CSRC + "rq_halves.hip", _CSRC + "rq_fast_common.h", _CSRC + "wave_ops.h", _CSRC + "device_common.h",
                  _CSRC + "internal.h")
GENERIC_SOURCES = (_CSRC + "rq_generic.hip", _CSRC + "device_common.h", _CSRC + "internal.h")
OUTER_SOURCES = (_CSRC + "rq_outer_impl.h", _CSRC + "rq_outer.hip", _CSRC + "rq_outer_t1.hip", _CSRC + "rq_outer_t2.hip",
                 _CSRC + "rq_outer_t4.hip", _CSRC + "rq_outer_t8.hip", _CSRC + "rq_outer_t16.hip", _CSRC + "wave_ops.h",
                 _CSRC + "device_common.h", _CSRC + "internal.h")
TRAFFIC_PROFILE = "profiles/{kernel}_n{n}_t{t}_hbm_traffic.txt"


def kernel_sources(kernel: str):
    return {"rq_generic": GENERIC_SOURCES, "rq_outer_mfma": OUTER_SOURCES,
            "rq_mfma28x2_w7": HALVES_SOURCES}.get(kernel, KERNEL_SOURCES)


def kernel_source_digest(kernel: str = "") -> str:
    """sha256 over the kernel's sources and the compile flags."""
    import hashlib

    from rotation_activation_quantization_amd import build as b

    h = hashlib.sha256()
    for p in kernel_sources(kernel):
        with open(os.path.join(HERE, p), "rb") as f:
            h.update(f.read())
    h.update(" ".join(b.COMMON).encode())
    return h.hexdigest()


def measured_traffic(kernel: str, n: int, t: int):
    """HBM bytes per launch from the committed counter summary (FETCH_SIZE and
    WRITE_SIZE, each scaled by what the counter reads for a plain copy of
    known size), or None if there is none or the kernel has changed since."""
    path = os.path.join(HERE, TRAFFIC_PROFILE.format(kernel=kernel, n=n, t=t))
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for ln in f:
            if "=" in ln and not ln.startswith("#"):
                k, v = ln.strip().split("=", 1)
                kv[k] = v
    if kv.get("source_sha256") != kernel_source_digest(kernel):
        return None
    return float(kv["traffic_bytes_per_launch"])


def algorithmic_bytes_per_token(n: int) -> int:
    # bf16 input + packed int4 codes + fp32 scale + fp32 zero-point
    return 2 * n + n // 2 + 8


def cpu_baseline(bits: np.ndarray, d: np.ndarray, per_config: dict | None = None) -> dict:
    """Time the oracle (numpy float64, as it stands) on a bounded sample of the
    same workload: one call over the first tokens of the batch (up to 8192
    at n <= 14336, 2048 above), so the oracle builds its column blocks of H
    once and the float64 product dominates.  per_config: {name: (first rows
    of that configuration's batch, its d)}, each timed the same way."""
    import oracle as O

    threads, blas = os.cpu_count() or 1, None
    try:
        from threadpoolctl import threadpool_info

        pools = [i for i in threadpool_info() if i.get("user_api") == "blas"] or threadpool_info()
        threads = max((i.get("num_threads", 1) for i in pools), default=threads)
        blas = ", ".join(sorted({f"{i.get('internal_api')} {i.get('version')}" for i in pools})) or None
    except Exception:  # pragma: no cover
        pass

    def timed(b, dd):
        t0 = time.perf_counter()
        O.rotate_quant_int4(b, dd)
        return time.perf_counter() - t0

    n = bits.shape[1]
    tokens = min(bits.shape[0], 8192 if n <= 14336 else 2048)
    dt = timed(bits[:tokens], d)
    out = {"value": tokens / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle", "blas": blas,
           "sample": f"the first {tokens} tokens of the same workload (n={n}) in one oracle call: float64 "
                     f"dense rotation built from column blocks of H (H construction included) + asymmetric "
                     f"INT4, {dt:.1f} s"}
    if per_config:
        out["per_config"] = {}
        for name, (b, dd) in per_config.items():
            t = timed(b, dd)
            out["per_config"][name] = {"value": b.shape[0] / t, "unit": "tokens/s", "sample_tokens": b.shape[0],
                                       "n": b.shape[1], "seconds": t}
    return out


def bench_fold(args, torch, R, W) -> int:
    """The offline weight fold on the LLaMA3-8B down-projection shape: W is
    [4096 output features, 14336] bf16 (synthetic N(0, 1/n)), d from the same
    calibration as the activations.  One step = one fold of the whole W."""
    rows, n = 4096, 14336
    g = torch.Generator(device="cpu").manual_seed(2611)
    w = (torch.randn((rows, n), generator=g) / n ** 0.5).to(torch.bfloat16).cuda()
    d = R.calibrate(to_dev_bits(W.calibration_batch("n14336_t8192")[0], torch))[0]
    out = torch.empty((rows, n), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    fn = R.lib().signrot_fold_weights
    sptr = ctypes.c_void_p(stream.cuda_stream)

    def step():
        st = fn(w.data_ptr(), rows, n, n, d.data_ptr(), out.data_ptr(), sptr)
        if st != 0:
            R.check(st, "signrot_fold_weights")

    for _ in range(args.warmup):
        step()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    bpr = 2 * n + 4 * n  # bf16 row in, fp32 row out
    achieved = bpr * rows / (ms * 1e-3) / 1e9
    line = {
        "metric": "weight rows/s and achieved HBM GB/s, SignRot offline weight fold W' = W.H.D/sqrt(n)",
        "value": rows * args.steps / wall, "unit": "rows/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"W {rows} x {n} bf16 N(0,1/n) (LLaMA3-8B down_proj shape) -> W' fp32",
                   "kernel": R.kernel_name(n),
                   "note": "the rotation kernels also write INT4 codes to a stream-ordered scratch "
                           f"({n // 2 + 8} B/row, not counted)"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": None, "bytes_per_row": bpr,
                     "kernel_avg_ms": ms},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_fold(w, d)
    print(json.dumps(line), flush=True)
    return 0


def cpu_baseline_fold(w, d, budget_s: float = 12.0) -> dict:
    """The oracle's fold_weights (float64 dense rotation) on 64-row chunks of
    the same W, for about budget_s seconds."""
    import torch

    import oracle as O

    wb = w.view(torch.int16).cpu().numpy().view(np.uint16)
    dn = d.cpu().numpy()
    chunk, done = 64, 0
    t0 = time.perf_counter()
    while done + chunk <= wb.shape[0]:
        O.fold_weights(wb[done:done + chunk], dn)
        done += chunk
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    try:
        from threadpoolctl import threadpool_info

        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    return {"value": done / dt, "unit": "rows/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} rows of the same W (n={wb.shape[1]}), oracle fold_weights (float64 dense "
                      f"rotation), {dt:.1f} s"}


PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA


def bench_linear(args, torch, R, W) -> int:
    """The consumer product on the LLaMA3-8B down-projection shape: 8192 tokens
    of INT4 activations (codes, scale, zero from signrot_rotate_quant_int4 on
    the n = 14336 workload) times the folded weight W' [4096, 14336] bf16
    (synthetic N(0, 1/n), folded with the same d).  One step = one
    signrot_int4_linear call over the whole batch."""
    rows = 4096
    bits, _ = W.batch("n14336_t8192")
    t, n = bits.shape
    d = R.calibrate(to_dev_bits(W.calibration_batch("n14336_t8192")[0], torch))[0]
    codes, scale, zero = R.rotate_quant_int4(to_dev_bits(bits, torch), d)
    g = torch.Generator(device="cpu").manual_seed(2612)
    w = (torch.randn((rows, n), generator=g) / n ** 0.5).to(torch.bfloat16).cuda()
    wf = R.fold_weights(w, d).to(torch.bfloat16)
    del w
    rs = R.weight_rowsum(wf)
    out = torch.empty((t, rows), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    sptr = ctypes.c_void_p(stream.cuda_stream)
    fn = R.lib().signrot_int4_linear
    argv = (codes.data_ptr(), scale.data_ptr(), zero.data_ptr(), t, n, wf.data_ptr(), n, rs.data_ptr(), rows,
            out.data_ptr(), sptr)

    def step():
        st = fn(*argv)
        if st != 0:
            R.check(st, "signrot_int4_linear")

    def timed(body, steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(steps):
            body()
        e1.record(stream)
        torch.cuda.synchronize()
        return time.perf_counter() - t0, e0.elapsed_time(e1) / steps

    for _ in range(args.warmup):
        step()
    wall, ms = timed(step, args.steps)
    flops = 2.0 * t * n * rows
    achieved = flops / (ms * 1e-3) / 1e12
    # context: the library bf16 GEMM (hipBLASLt via torch) on the same shape,
    # alone (activations already dequantized to bf16) and as the unfused
    # consumer it would be here (dequantize to bf16, then the GEMM)
    yb = R.dequant(codes, scale, zero).to(torch.bfloat16)
    wt = wf.t()
    for _ in range(20):
        torch.matmul(yb, wt)
    _, ms_lib = timed(lambda: torch.matmul(yb, wt), 50)
    del yb
    _, ms_unfused = timed(lambda: torch.matmul(R.dequant(codes, scale, zero).to(torch.bfloat16), wt), 20)
    line = {
        "metric": "tokens/s and achieved TFLOP/s, INT4-activation down-projection with zero-point correction",
        "value": t * args.steps / wall, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16 x u4 -> f32", "data": "synthetic",
        "config": {"workload": f"{t} tokens x n={n} INT4 codes (n=14336 workload, quantized on the GPU) "
                               f"times W' [{rows} x {n}] bf16, out f32 [{t} x {rows}]",
                   "kernel": R.int4_linear_kernel_name(codes, wf),
                   "library_bf16_gemm_ms": ms_lib,
                   "library_bf16_gemm_tflops": flops / (ms_lib * 1e-3) / 1e12,
                   "unfused_dequant_plus_library_gemm_ms": ms_unfused},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None, "flops_per_launch": flops,
                     "kernel_avg_ms": ms},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_linear(codes, scale, zero, wf)
    print(json.dumps(line), flush=True)
    return 0


def bench_swiglu(args, torch, R, W) -> int:
    """The online path with the SwiGLU producer fused in, on the named
    workload's law (default n = 14336 at 8192 tokens): gate and up bf16
    [T, n] (seeded synthetic, the massive channel in the workload's outlier
    tokens), d calibrated on x of a 256-token calibration batch.  One step =
    one signrot_swiglu_rotate_quant_int4 call (reads gate and up, writes
    codes).  Beside it, the unfused pair it replaces: the producer as a
    library elementwise kernel (torch, binary32 SiLU(gate) * up stored as
    bf16) and then signrot_rotate_quant_int4_outlier on that x."""
    gate_b, up_b, _ = W.swiglu_batch(args.workload, tokens=args.tokens)
    t, n = gate_b.shape
    cg, cu, _ = W.swiglu_batch(args.workload, tokens=256, stream=11)
    stream = torch.cuda.current_stream()
    g0, u0 = to_dev_bits(gate_b, torch), to_dev_bits(up_b, torch)
    del gate_b, up_b
    xcal = (torch.nn.functional.silu(to_dev_bits(cg, torch).float()) * to_dev_bits(cu, torch).float()).bfloat16()
    _, c, _, mc = R.calibrate(xcal)
    sigma = -1 if mc < 0 else 1
    nsets = max(2, int(np.ceil(BUFFER_SETS_MIN_BYTES / (4 * t * n))))
    gs = [g0] + [g0.clone() for _ in range(nsets - 1)]
    us = [u0] + [u0.clone() for _ in range(nsets - 1)]
    xs = [torch.empty((t, n), dtype=torch.bfloat16, device="cuda") for _ in range(nsets)]
    outs = [(torch.empty((t, n // 2), dtype=torch.uint8, device="cuda"), torch.empty(t, device="cuda"),
             torch.empty(t, device="cuda")) for _ in range(nsets)]
    sptr = ctypes.c_void_p(stream.cuda_stream)
    L = R.lib()

    def fused(i):
        k = i % nsets
        st = L.signrot_swiglu_rotate_quant_int4(gs[k].data_ptr(), us[k].data_ptr(), t, n, n, c, sigma,
                                                outs[k][0].data_ptr(), outs[k][1].data_ptr(),
                                                outs[k][2].data_ptr(), None, sptr)
        if st != 0:
            R.check(st, "signrot_swiglu_rotate_quant_int4")

    def producer_into(i):
        k = i % nsets
        xs[k].copy_(torch.nn.functional.silu(gs[k].float()).mul_(us[k].float()))

    def rotate(i):
        k = i % nsets
        st = L.signrot_rotate_quant_int4_outlier(xs[k].data_ptr(), t, n, n, c, sigma, outs[k][0].data_ptr(),
                                                 outs[k][1].data_ptr(), outs[k][2].data_ptr(), None, sptr)
        if st != 0:
            R.check(st, "signrot_rotate_quant_int4_outlier")

    for i in range(nsets):
        producer_into(i)
    unf_rot = leg(torch, stream, rotate, 100, 200)
    unf_prod = leg(torch, stream, producer_into, 20, 50)
    for i in range(args.warmup):
        fused(i)
    head = timed_launches(torch, stream, fused, args.steps)
    ms = head["mean_ms"]
    fused_bytes = t * (4 * n + n // 2 + 8)  # gate + up in, codes + scale + zero out
    achieved = fused_bytes / (ms * 1e-3) / 1e9
    line = {
        "metric": "tokens/s and achieved HBM GB/s, SignRot rotate+INT4 with the SwiGLU producer fused in",
        "value": t * args.steps / head["wall_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": head["wall_s"] * 1e3 / args.steps, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"gate, up bf16 [{t} x {n}] (gate N(0,1.5), up N(0,0.6); massive channel {c} "
                               f"in {100 * W.WORKLOADS[args.workload].p_outlier:.0f}% of tokens), "
                               "x = bf16(SiLU(gate) * up) in the kernel",
                   "kernel": R.kernel_name(n) + " (SwiGLU instance)",
                   "launch_ms": {k: head[k] for k in ("mean_ms", "p10_ms", "p50_ms", "p90_ms", "group")},
                   "unfused_producer_ms": unf_prod["mean_ms"],
                   "unfused_rotate_ms": unf_rot["mean_ms"],
                   "unfused_total_ms": unf_prod["mean_ms"] + unf_rot["mean_ms"],
                   "hbm_bytes_fused": fused_bytes,
                   "hbm_bytes_unfused": t * (4 * n + 2 * n) + t * (2 * n + n // 2 + 8)},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": None, "bytes_per_token": 4 * n + n // 2 + 8,
                     "kernel_avg_ms": ms},
    }
    print(json.dumps(line), flush=True)
    return 0


def cpu_baseline_linear(codes, scale, zero, wf, budget_s: float = 12.0) -> dict:
    """The oracle's int4_linear (float64 dequantize, then numpy matmul) on
    32-token chunks of the same operands, for about budget_s seconds."""
    import oracle as O

    c = codes.cpu().numpy()
    s = scale.cpu().numpy()
    z = zero.cpu().numpy()
    wb = wf.view(torch_int16()).cpu().numpy().view(np.uint16)
    chunk, done = 32, 0
    t0 = time.perf_counter()
    while done + chunk <= c.shape[0]:
        O.int4_linear(c[done:done + chunk], s[done:done + chunk], z[done:done + chunk], wb)
        done += chunk
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    try:
        from threadpoolctl import threadpool_info

        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    return {"value": done / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} tokens x {wb.shape[0]} rows of the same operands, oracle int4_linear "
                      f"(float64 dequantize + matmul), {dt:.1f} s"}


def torch_int16():
    import torch

    return torch.int16


def workload_text(w, n: int, t: int, c: int) -> str:
    width = {4096: "2^12", 8192: "2^13", 14336: "28*2^9, LLaMA3-8B down_proj input",
             28672: "28*2^10, LLaMA3-70B down_proj input",
             11008: "344*2^5, Paley I over GF(7^3), LLaMA-2-7B down_proj input"}.get(n, str(n))
    law = f"N(0,{w.width:g})" if w.law == "normal" else f"{w.width:g}*t({w.df:g})"
    sign = "+" if w.p_positive >= 1.0 else f"+-(+ {w.p_positive:.0%})"
    mild = f", {w.mild_channels} mild channels x{w.mild_factor:g}" if w.mild_channels else ""
    cal = "the batch itself" if w.calib_same else f"{w.calib_tokens} tokens"
    return (f"n={n} ({width}) x {t} tokens bf16, {law} background{mild}, outlier channel {c} with "
            f"{sign}M, M~U[{w.m_lo:g},{w.m_hi:g}] in {w.p_outlier:.0%} of tokens; SignRot sign vector from "
            f"calibration on {cal}")


def decode_latency(R, W, torch, c, sigma, calls: int = 10000) -> dict:
    """Latency of decode-shaped calls (1, 4, 16 tokens of the n = 14336 law):
    microseconds per call for back-to-back launches and for one HIP graph
    holding `calls` launches.  The graph's output is checked against an eager
    call on the same input after every replay."""
    out = {}
    fn = R.lib().signrot_rotate_quant_int4_outlier
    for t in (1, 4, 16):
        bits, _ = W.decode_batch("n14336_decode", t, 0)
        n = bits.shape[1]
        x = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
        co = torch.empty((t, n // 2), dtype=torch.uint8, device="cuda")
        sc = torch.empty(t, dtype=torch.float32, device="cuda")
        ze = torch.empty(t, dtype=torch.float32, device="cuda")
        ref = R.rotate_quant_int4_outlier(x, c, sigma)

        def launch(stream):
            st = fn(x.data_ptr(), t, n, n, c, sigma, co.data_ptr(), sc.data_ptr(), ze.data_ptr(), None,
                    ctypes.c_void_p(stream.cuda_stream))
            if st != 0:
                R.check(st, "signrot_rotate_quant_int4_outlier")

        stream = torch.cuda.current_stream()
        for _ in range(100):
            launch(stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(calls):
            launch(stream)
        e1.record(stream)
        torch.cuda.synchronize()
        us_launch = e0.elapsed_time(e1) * 1e3 / calls

        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                cap = torch.cuda.current_stream()
                for _ in range(calls):
                    launch(cap)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        times = []
        for rep in range(3):
            co.zero_()
            torch.cuda.synchronize()
            e0.record(stream)
            g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e3 / calls)
            if not (torch.equal(co, ref[0]) and torch.equal(sc, ref[1]) and torch.equal(ze, ref[2])):
                raise RuntimeError(f"graph replay {rep} differs from the eager call at {t} tokens")
        del g
        out[str(t)] = {"us_per_call_launch": us_launch, "us_per_call_graph": float(np.median(times))}
    return out


def timed_launches(torch, stream, launch, steps: int, group: int = 10) -> dict:
    """Run launch(i) for i < steps with HIP events recorded on `stream`: one
    before the first launch and one after every `group` launches (and after
    the last).  The mean launch time is (last event - first) / steps; the
    10th / 50th / 90th percentiles are over the per-launch means of the
    groups, so that no event sits between every two launches (an event per
    launch adds a few microseconds to each).  Times in ms, plus the wall
    time of the region in s."""
    marks = list(range(group, steps, group)) + [steps]
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(marks) + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record(stream)
    k = 0
    for i in range(steps):
        launch(i)
        if i + 1 == marks[k]:
            k += 1
            evs[k].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    bounds = [0] + marks
    per = np.array([evs[j].elapsed_time(evs[j + 1]) / (bounds[j + 1] - bounds[j]) for j in range(len(marks))])
    return {"mean_ms": evs[0].elapsed_time(evs[-1]) / steps, "p10_ms": float(np.percentile(per, 10)),
            "p50_ms": float(np.percentile(per, 50)), "p90_ms": float(np.percentile(per, 90)),
            "group": group, "wall_s": wall}


def leg(torch, stream, launch, warmup: int, steps: int) -> dict:
    for i in range(warmup):
        launch(i)
    r = timed_launches(torch, stream, launch, steps)
    r.pop("wall_s")
    return r


def paired_legs(torch, stream, launch_a, launch_b, rounds: int = 8, group: int = 50) -> dict:
    """Two entry points in alternating groups of `group` launches (a, b, a,
    b, ...), so that both see the same clock: the mean launch time of each
    (ms) and their difference (us), with the per-round differences."""
    ta, tb = [], []
    for _ in range(rounds):
        ta.append(timed_launches(torch, stream, launch_a, group, group)["mean_ms"])
        tb.append(timed_launches(torch, stream, launch_b, group, group)["mean_ms"])
    diff = [1e3 * (b - a) for a, b in zip(ta, tb)]
    return {"a_mean_ms": float(np.mean(ta)), "b_mean_ms": float(np.mean(tb)),
            "b_minus_a_us": float(np.mean(diff)), "b_minus_a_us_per_round": [round(x, 3) for x in diff],
            "rounds": rounds, "group": group}


def mse_summary(torch, R, x, c, sigma, outlier_tokens, n: int) -> dict:
    """Quantization MSE of the GPU's own outputs on the first 1024 tokens, in
    the rotated domain: mean over channels of (y - dequant(codes))^2 with y
    the kernel's binary32 rotated values, for SignRot (d = sigma * row c of
    H) and for plain Hadamard (d = all ones), both asymmetric INT4, split into
    tokens with and without the outlier.  Beside it, the oracle's stored grid
    (tests/golden/mse_grid.json, written offline by the oracle) for every
    configuration and the decode control batch, which also holds the
    symmetric-INT4 cells."""
    t = min(1024, x.shape[0])
    xs = x[:t]
    out = np.zeros(t, bool)
    out[outlier_tokens[outlier_tokens < t]] = True
    res = {"tokens": t, "outlier_tokens": int(out.sum())}
    ones = torch.ones(n, dtype=torch.int8, device=x.device)
    for name, call in (("signrot_asym", lambda: R.rotate_quant_int4_outlier(xs, c, sigma, y_out=True)),
                       ("plain_asym", lambda: R.rotate_quant_int4(xs, ones, y_out=True))):
        codes, scale, zero, y = call()
        yh = R.dequant(codes, scale, zero)
        m = ((y.double() - yh.double()) ** 2).mean(dim=1).cpu().numpy()
        res[name] = {"outlier": float(m[out].mean()) if out.any() else None,
                     "no_outlier": float(m[~out].mean()) if (~out).any() else None}
        del codes, scale, zero, y, yh
    path = os.path.join(HERE, "tests", "golden", "mse_grid.json")
    if os.path.exists(path):
        with open(path) as f:
            res["oracle_grid"] = json.load(f)["workloads"]
    return res


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--tokens", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pmc-copy", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--fold", action="store_true",
                    help="time the offline weight fold W' = W.H.D/sqrt(n) instead (W: 4096 x 14336 bf16)")
    ap.add_argument("--linear", action="store_true",
                    help="time the INT4-activation down-projection signrot_int4_linear instead "
                         "(8192 x 14336 codes, W' 4096 x 14336 bf16)")
    ap.add_argument("--swiglu", action="store_true",
                    help="time the online path with the SwiGLU producer fused in (gate, up 8192 x 14336 bf16) "
                         "against the unfused producer + rotate pair")
    ap.add_argument("--workload", default=WORKLOAD,
                    choices=["n4096_t64", "n8192_t2048", "n14336_t4096", "n14336_t8192", "n28672_t8192",
                             "n11008_t8192"],
                    help="synthetic workload to time (default: n=14336 x 8192 tokens)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for --gpus {args.gpus}); "
              "tokens shard across GPUs with no exchange between them (each GPU rotates and quantizes its own rows).",
              file=sys.stderr)
        return 2

    import torch

    import rotation_activation_quantization_amd as R
    import signrot_workloads as W

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    if args.fold:
        return bench_fold(args, torch, R, W)
    if args.linear:
        return bench_linear(args, torch, R, W)
    if args.swiglu:
        return bench_swiglu(args, torch, R, W)
    L = R.lib()

    wname = args.workload
    w = W.WORKLOADS[wname]
    bits, meta = W.batch(wname, tokens=args.tokens)
    t, n = bits.shape
    x0 = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    d, c, _, mc = R.calibrate(to_dev_bits(W.calibration_batch(wname)[0], torch))
    sigma = -1 if mc < 0 else 1

    in_bytes = x0.numel() * 2
    nsets = max(2, int(np.ceil(BUFFER_SETS_MIN_BYTES / in_bytes)))
    xs = [x0] + [x0.clone() for _ in range(nsets - 1)]
    outs = [(torch.empty((t, n // 2), dtype=torch.uint8, device="cuda"),
             torch.empty(t, dtype=torch.float32, device="cuda"),
             torch.empty(t, dtype=torch.float32, device="cuda")) for _ in range(nsets)]
    stream = torch.cuda.current_stream()
    sptr = ctypes.c_void_p(stream.cuda_stream)
    # the step: the calibrated sign vector d = sigma * (row c of H), passed as
    # (c, sigma)
    calls = []
    for i in range(nsets):
        co, sc, ze = outs[i]
        calls.append((xs[i].data_ptr(), t, n, n, c, sigma, co.data_ptr(), sc.data_ptr(), ze.data_ptr(),
                      None, sptr))
    fn = L.signrot_rotate_quant_int4_outlier

    def step(i):
        st = fn(*calls[i % nsets])
        if st != 0:
            R.check(st, "signrot_rotate_quant_int4_outlier")

    # Auxiliary legs first, each with a warm-up of its own: the traffic
    # ceiling, the d-vector entry point and the integer zero-point variant on
    # the same buffers.
    dcalls = [(xs[i].data_ptr(), t, n, n, d.data_ptr(), outs[i][0].data_ptr(), outs[i][1].data_ptr(),
               outs[i][2].data_ptr(), None, sptr) for i in range(nsets)]

    def dstep(i):
        st = L.signrot_rotate_quant_int4(*dcalls[i % nsets])
        if st != 0:
            R.check(st, "signrot_rotate_quant_int4")

    def zstep(i):
        co, sc, ze = outs[i % nsets]
        st = L.signrot_rotate_quant_int4_zint(xs[i % nsets].data_ptr(), t, n, n, c, sigma, co.data_ptr(),
                                             sc.data_ptr(), ze.data_ptr(), sptr)
        if st != 0:
            R.check(st, "signrot_rotate_quant_int4_zint")

    def cstep(i):
        co, sc, ze = outs[i % nsets]
        st = L.signrot_stream_ceiling(xs[i % nsets].data_ptr(), t, n, n, co.data_ptr(), sc.data_ptr(),
                                      ze.data_ptr(), sptr)
        if st != 0:
            R.check(st, "signrot_stream_ceiling")

    # The GPU's clock settles over the first tens of milliseconds under load:
    # a leg timed right after start-up ran up to 10 % slow.  So every leg
    # below is timed after a quarter of a second of headline launches.
    warm_end = time.perf_counter() + 0.25
    i = 0
    while time.perf_counter() < warm_end:
        for _ in range(32):
            step(i)
            i += 1
        torch.cuda.synchronize()

    aux_steps = 200
    ceiling = leg(torch, stream, cstep, 100, aux_steps)
    dvec = leg(torch, stream, dstep, 100, aux_steps)
    zint = leg(torch, stream, zstep, 100, aux_steps)
    # the d-vector entry point against the headline's (c, sigma) one under the
    # same clock (before the headline's warm-up, so that the last launches of
    # the process are the timed ones)
    dpair = paired_legs(torch, stream, step, dstep)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # HIP events on the stream the kernel is launched on, one before the
    # first timed step and one after every ten steps: the average launch
    # duration is (last - first) / steps, and the ten-launch means give the
    # percentiles.  synchronize() brackets the timed region on both sides.
    head = timed_launches(torch, stream, step, args.steps)
    wall = head["wall_s"]
    avg_kernel_ms = head["mean_ms"]

    if args.pmc_copy:
        # plain copies of known size, for scaling rocprofv3 FETCH_SIZE/WRITE_SIZE
        src = torch.empty(256 * 2**20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()

    ms_per_step = wall * 1e3 / args.steps
    tokens_per_s = t * args.steps / wall
    bpt = algorithmic_bytes_per_token(n)
    achieved = bpt * t / (avg_kernel_ms * 1e-3) / 1e9
    kname = R.kernel_name(n)
    ceiling_gbs = bpt * t / (ceiling["mean_ms"] * 1e-3) / 1e9
    traffic_bytes = measured_traffic(kname, n, t)
    traffic = None if traffic_bytes is None else traffic_bytes / (avg_kernel_ms * 1e-3) / 1e9
    line = {
        "metric": "tokens/s and achieved HBM GB/s (% of peak), fused SignRot rotate+INT4 quant",
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": workload_text(w, n, t, c),
            "n": n,
            "tokens": t,
            "parallelism": "single GPU",
            "kernel": kname,
            "entry_point": "signrot_rotate_quant_int4_outlier (d = sigma * row c of H, from calibration)",
            "d_vector_entry_point_kernel_avg_ms": dvec["mean_ms"],
            "d_vector_entry_point_launch_ms": dvec,
            "d_vector_minus_c_sigma_paired": {
                "c_sigma_mean_ms": dpair["a_mean_ms"], "d_vector_mean_ms": dpair["b_mean_ms"],
                "difference_us": dpair["b_minus_a_us"], "per_round_us": dpair["b_minus_a_us_per_round"],
                "launches": f"{dpair['rounds']} rounds of {dpair['group']} + {dpair['group']}, alternating, before "
                            "the headline's warm-up"},
            "integer_zero_point_variant_kernel_avg_ms": zint["mean_ms"],
            "integer_zero_point_variant_launch_ms": zint,
            "launch_ms": {k: head[k] for k in ("mean_ms", "p10_ms", "p50_ms", "p90_ms", "group")},
            "aux_legs": f"{aux_steps} launches each after 100 warm-up, run before the headline steps and after 0.25 s "
                        "of untimed headline launches (steady clock)",
            "input_buffer_sets": nsets,
            "hbm_gbs_wall": bpt * tokens_per_s / 1e9,
            "pct_of_peak_hbm_wall": 100.0 * bpt * tokens_per_s / 1e9 / PEAK_HBM_GBS,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS,
            "traffic": traffic,
            "traffic_bytes_per_launch": traffic_bytes,
            "algorithmic_bytes_per_launch": bpt * t,
            "bytes_per_token": bpt,
            "kernel_avg_ms": avg_kernel_ms,
            "ceiling": {"kernel": "signrot_stream_ceiling (the path's bytes per token, no arithmetic)",
                        "achieved": ceiling_gbs, "frac_of_peak": ceiling_gbs / PEAK_HBM_GBS,
                        "launch_ms": ceiling},
            "frac_of_ceiling": achieved / ceiling_gbs,
        },
    }
    line["mse"] = mse_summary(torch, R, x0, c, sigma, meta["outlier_tokens"], n)
    if not args.no_decode and n == 14336:
        line["decode"] = {"workload": "n=14336, 1/4/16 tokens per call, same law; 10^4 calls",
                          "tokens": decode_latency(R, W, torch, c, sigma)}
    if not args.no_decode and wname == WORKLOAD and args.tokens is None:
        del xs, outs, calls, dcalls
        torch.cuda.empty_cache()
        samples = {}
        line["other_configs"] = {}
        for name in OTHER_CONFIGS:
            line["other_configs"][name], samples[name] = config_leg(R, W, torch, L, name)
    else:
        samples = None
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(bits, d.cpu().numpy(), samples)
    print(json.dumps(line), flush=True)
    return 0


OTHER_CONFIGS = ("n4096_t64", "n8192_t2048", "n14336_t4096", "n28672_t8192")
# rows of each configuration's batch kept for the oracle's CPU timing
CPU_SAMPLE_ROWS = {"n4096_t64": 64, "n8192_t2048": 2048, "n14336_t4096": 4096, "n28672_t8192": 1024}


def config_leg(R, W, torch, L, name: str, warmup: int = 100, steps: int = 200):
    """One more configuration on the (c, sigma) entry point: its own synthetic
    batch and calibration, input copies rotated so that each launch reads
    HBM (at most 64 copies: the 64-token batch stays cache-resident and is
    launch-bound), the traffic-ceiling kernel on the same buffers first.
    Returns the record and (the batch's first rows, d) for the CPU timing."""
    bits, _ = W.batch(name)
    t, n = bits.shape
    x0 = to_dev_bits(bits, torch)
    d, c, _, mc = R.calibrate(to_dev_bits(W.calibration_batch(name)[0], torch))
    sigma = -1 if mc < 0 else 1
    nsets = min(64, max(2, int(np.ceil(BUFFER_SETS_MIN_BYTES / (x0.numel() * 2)))))
    xs = [x0] + [x0.clone() for _ in range(nsets - 1)]
    outs = [(torch.empty((t, n // 2), dtype=torch.uint8, device="cuda"),
             torch.empty(t, dtype=torch.float32, device="cuda"),
             torch.empty(t, dtype=torch.float32, device="cuda")) for _ in range(nsets)]
    stream = torch.cuda.current_stream()
    sptr = ctypes.c_void_p(stream.cuda_stream)

    def step(i):
        co, sc, ze = outs[i % nsets]
        st = L.signrot_rotate_quant_int4_outlier(xs[i % nsets].data_ptr(), t, n, n, c, sigma, co.data_ptr(),
                                                 sc.data_ptr(), ze.data_ptr(), None, sptr)
        if st != 0:
            R.check(st, "signrot_rotate_quant_int4_outlier")

    def cstep(i):
        co, sc, ze = outs[i % nsets]
        st = L.signrot_stream_ceiling(xs[i % nsets].data_ptr(), t, n, n, co.data_ptr(), sc.data_ptr(),
                                      ze.data_ptr(), sptr)
        if st != 0:
            R.check(st, "signrot_stream_ceiling")

    ceiling = leg(torch, stream, cstep, warmup, steps)
    run = leg(torch, stream, step, warmup, steps)
    bpt = algorithmic_bytes_per_token(n)
    gbs = bpt * t / (run["mean_ms"] * 1e-3) / 1e9
    ceil_gbs = bpt * t / (ceiling["mean_ms"] * 1e-3) / 1e9
    out = {"n": n, "tokens": t, "kernel": R.kernel_name(n), "tokens_per_s": t / (run["mean_ms"] * 1e-3),
           "launch_ms": run, "achieved_gbs": gbs, "frac_of_peak": gbs / PEAK_HBM_GBS,
           "ceiling_launch_ms": ceiling, "ceiling_frac_of_peak": ceil_gbs / PEAK_HBM_GBS,
           "frac_of_ceiling": gbs / ceil_gbs, "input_buffer_sets": nsets,
           "launches": f"{warmup} warm-up + {steps} timed each, ceiling first"}
    del xs, outs
    torch.cuda.empty_cache()
    return out, (np.ascontiguousarray(bits[:CPU_SAMPLE_ROWS[name]]), d.cpu().numpy())


def to_dev_bits(bits, torch):
    t, n = bits.shape
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


if __name__ == "__main__":
    sys.exit(main())
