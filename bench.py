#!/usr/bin/env python3
"""Benchmark of the FP8 group-quantize + block-scaled GEMM path on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic inputs, for every linear of the
workload: 128x128 block quantization of the bf16 master weights (with the transposed copy), 1x128 and
128x1 (transposed) quantization of X from one read, the forward GEMM, 1x128 and 128x1 quantization of dY
from one read, DGrad, WGrad.  --separate-quant runs the 1x128 and 128x1 quantizers as separate kernels
(two reads of X and of dY) instead; the codes and scales are the same bits either way.  Inputs are generated on the GPU and resident in HBM before timing starts; outputs
are preallocated.  The headline value is GEMM TFLOP/s over the whole step (GEMM flops / step time,
quantization included).

Prints one JSON line.  Besides the contract fields it carries
  roofline      the GEMM kernel: algorithmic flops (2*M*N*K per launch) / mean launch time, measured with
                HIP events on the launch stream over the timed steps, against the MI355X dense FP8 peak;
                traffic = HBM bytes per launch from rocprofv3 counters when supplied (--traffic-json).
  roofline_quant the quantize kernels: algorithmic bytes / time against 8 TB/s.
  cpu_baseline  the CPU oracle timed on this host on a bounded sample of the same workload.

--producers prints a separate line for the fused producers that emit 1x128 FP8 directly (RMSNorm and SwiGLU):
algorithmic bytes (bf16 read, codes and scales written, rstd) / kernel time against 8 TB/s, per kernel.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FP8_PEAK_TFLOPS = 5000.0      # MI355X dense FP8 matrix peak
HBM_PEAK_GBS = 8000.0         # MI355X HBM3E
METRIC = "block-scaled FP8 GEMM TFLOP/s (fwd+dgrad+wgrad), % of MI355X FP8 peak"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="qwen25_32b_train_m65536",
                   help="training-step workload (default: the Qwen2.5-32B-shaped linears at 65536 tokens, the largest "
                        "single-GPU configuration; llama3_8b_train_m16384 is the 8B step at 16384 tokens)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample-rows", type=int, default=None,
                   help="token rows per linear of the oracle's all-thread sample (default: 64 for the 32B shapes, "
                        "128 otherwise); the one-thread sample uses 1/16 of them")
    p.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "gemm_traffic.json"),
                   help="per-launch HBM bytes measured by rocprofv3 for this workload (optional)")
    p.add_argument("--x-from-fp8", action="store_true",
                   help="WGrad's X from the saved 1x128 FP8 codes (dequantize, requantize 128x1) instead of bf16 X")
    p.add_argument("--separate-quant", action="store_true",
                   help="quantize X and dY with the 1x128 and 128x1 kernels separately (two reads each)")
    p.add_argument("--producers", action="store_true",
                   help="instead of the GEMM step, time the fused producers of one layer (2 RMSNorm -> 1x128 and "
                        "1 SwiGLU -> 1x128 at the workload's token count) and print their own JSON line")
    p.add_argument("--decode", action="store_true",
                   help="instead of the training step, time rollout decode (workload llama3_8b_decode_m32: per step the "
                        "tokens' 1x128 activation quantization and the forward GEMM of the four linears against FP8 "
                        "weights quantized beforehand) and print its own JSON line")
    p.add_argument("--decode-rows", type=int, default=None,
                   help="token rows of a decode step (default: the workload's 32)")
    p.add_argument("--decode-rowmajor", action="store_true",
                   help="decode over row-major FP8 weights (jetfp8_gemm_fwd) instead of the fragment order "
                        "(JETFP8_BLOCKS_128x128_FRAG + jetfp8_gemm_fwd_frag, used up to 64 rows)")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="first run a 1 GiB device-to-device copy (known bytes) to scale rocprofv3 byte counters")
    return p.parse_args()


CSRC = os.path.join(ROOT, "fp8_precision_rl_amd", "csrc")
GEMM_SOURCES = [os.path.join(CSRC, f) for f in ("jetfp8_gemm.hip", "jetfp8_mfma.h", "jetfp8_common.h")]
DECODE_SOURCES = [os.path.join(CSRC, f) for f in ("jetfp8_decode.hip", "jetfp8_mfma.h", "jetfp8_common.h")]


def source_digest(paths=GEMM_SOURCES) -> str:
    """sha256 over the kernel's source files with comments and blank lines removed: a traffic record applies only
    to the code it was taken on, and an edit of comments alone does not void it."""
    import hashlib
    import re
    text = "\n".join(open(p).read() for p in paths)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*", "", line).rstrip() for line in text.splitlines())
    return hashlib.sha256("\n".join(line for line in lines if line).encode()).hexdigest()


def recorded_traffic(path, workload):
    """HBM bytes per GEMM launch recorded from rocprofv3 FETCH_SIZE / WRITE_SIZE runs (scaled by a copy
    kernel of known size), or None when absent, for another workload, or taken on a different kernel."""
    try:
        tj = json.load(open(path))
    except (OSError, ValueError):
        return None
    if tj.get("workload") != workload or tj.get("kernel_source_sha256") != source_digest():
        return None
    return tj.get("gemm_bytes_per_launch")


def copy_calibration(torch):
    """1 GiB uint8 device copy, twice: reads and writes exactly 2^30 bytes per launch."""
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


class Linear:
    """Device buffers of one FP8 linear layer for a full training step."""

    def __init__(self, wl, index, torch, workloads):
        d = workloads.device_linear(wl, index)
        self.name, self.M, self.K, self.N = d["name"], d["M"], d["K"], d["N"]
        M, K, N = self.M, self.K, self.N
        dev = d["x"].device
        u8, f32, bf = torch.uint8, torch.float32, torch.bfloat16
        self.x, self.w, self.dy = d["x"], d["w"], d["dy"]
        self.wq = torch.empty((N, K), dtype=u8, device=dev)
        self.wqT = torch.empty((K, N), dtype=u8, device=dev)
        self.ws = torch.empty((N // 128, K // 128), dtype=f32, device=dev)
        self.xq = torch.empty((M, K), dtype=u8, device=dev)
        self.xs = torch.empty((K // 128, M), dtype=f32, device=dev)
        self.y = torch.empty((M, N), dtype=bf, device=dev)
        self.dyq = torch.empty((M, N), dtype=u8, device=dev)
        self.dys = torch.empty((N // 128, M), dtype=f32, device=dev)
        self.dx = torch.empty((M, K), dtype=bf, device=dev)
        self.dyqT = torch.empty((N, M), dtype=u8, device=dev)
        self.dysT = torch.empty((M // 128, N), dtype=f32, device=dev)
        self.xqT = torch.empty((K, M), dtype=u8, device=dev)
        self.xsT = torch.empty((M // 128, K), dtype=f32, device=dev)
        self.dw = torch.empty((N, K), dtype=bf, device=dev)

    def gemm_flops(self):
        return 3 * 2 * self.M * self.N * self.K

    def quant_bytes(self):
        M, N, K = self.M, self.N, self.K
        rows = 2 + 1 + 4 / 128                      # bf16 in, code out, one fp32 scale per 128
        dual = 2 + 2 + 8 / 128                      # bf16 in, both codes out, both scales
        requant = 1 + 1 + 8 / 128                   # codes in, codes out, both scales
        return {"w_blocks_T": N * K * (2 + 1 + 1 + 4 / 16384), "x_rows": M * K * rows, "dy_rows": M * N * rows,
                "dy_cols_t": M * N * rows, "x_cols_t": M * K * rows, "x_dual": M * K * dual, "dy_dual": M * N * dual,
                "x_requant_t": M * K * requant}


def run_step(L, jf, st, ev=None, fused=True, x_from_fp8=False):
    """One pass of the hot path over one linear.  ev: optional list collecting (kind, name, flops_or_bytes,
    start_event, end_event) around each launch.  fused: X and dY are quantized in both groupings by one
    kernel each (one read); otherwise by the 1x128 and the 128x1 kernels separately.  x_from_fp8: WGrad's X
    operand is requantized from the saved 1x128 FP8 codes of X instead of from bf16 X."""
    M, N, K = L.M, L.N, L.K

    def timed(kind, name, amount, fn):
        if ev is None:
            fn()
            return
        import torch
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        ev.append((kind, name, amount, a, b))

    qb = L.quant_bytes()
    timed("quant", "w_blocks_T", qb["w_blocks_T"],
          lambda: jf.jetfp8_quantize(L.w, N, K, jf.BLOCKS_128x128, L.wq, L.ws, L.wqT, st))
    if fused and not x_from_fp8:
        timed("quant", "x_dual", qb["x_dual"],
              lambda: jf.jetfp8_quantize_dual(L.x, M, K, L.xq, L.xs, L.xqT, L.xsT, st))
    else:
        timed("quant", "x_rows", qb["x_rows"],
              lambda: jf.jetfp8_quantize(L.x, M, K, jf.ROWS_1x128, L.xq, L.xs, None, st))
    timed("gemm", "fwd", 2 * M * N * K, lambda: jf.jetfp8_gemm_fwd(L.xq, L.xs, L.wq, L.ws, L.y, M, N, K, st))
    if fused:
        timed("quant", "dy_dual", qb["dy_dual"],
              lambda: jf.jetfp8_quantize_dual(L.dy, M, N, L.dyq, L.dys, L.dyqT, L.dysT, st))
    else:
        timed("quant", "dy_rows", qb["dy_rows"],
              lambda: jf.jetfp8_quantize(L.dy, M, N, jf.ROWS_1x128, L.dyq, L.dys, None, st))
    timed("gemm", "dgrad", 2 * M * N * K, lambda: jf.jetfp8_gemm_dgrad(L.dyq, L.dys, L.wqT, L.ws, L.dx, M, N, K, st))
    if not fused:
        timed("quant", "dy_cols_t", qb["dy_cols_t"],
              lambda: jf.jetfp8_quantize(L.dy, M, N, jf.COLS_128x1_T, L.dyqT, L.dysT, None, st))
    if x_from_fp8:
        timed("quant", "x_requant_t", qb["x_requant_t"],
              lambda: jf.jetfp8_requantize_cols_t(L.xq, L.xs, M, K, L.xqT, L.xsT, st))
    elif not fused:
        timed("quant", "x_cols_t", qb["x_cols_t"],
              lambda: jf.jetfp8_quantize(L.x, M, K, jf.COLS_128x1_T, L.xqT, L.xsT, None, st))
    timed("gemm", "wgrad", 2 * M * N * K, lambda: jf.jetfp8_gemm_wgrad(L.dyqT, L.dysT, L.xqT, L.xsT, L.dw, M, N, K, st))


def step_description(args):
    x = ("X rows quant, fwd" if args.x_from_fp8 or args.separate_quant else "X rows+cols(T) quant in one read, fwd")
    dy = "dY rows quant, dgrad, dY cols quant (T)" if args.separate_quant else "dY rows+cols(T) quant in one read, dgrad"
    xt = ", X cols (T) requantized from the saved FP8 X" if args.x_from_fp8 else (
        ", X cols quant (T)" if args.separate_quant else "")
    return f"per linear: W block quant(+T), {x}, {dy}{xt}, wgrad"


def host_core_counts():
    """(logical CPUs of the host, CPUs this process may run on)."""
    n = os.cpu_count() or 1
    try:
        aff = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        aff = n
    return n, aff


def cpu_baseline(wl, rows, workloads):
    """The oracle (unchanged) on a bounded sample of the workload, timed twice on this host: with all the threads
    it uses by default (its pool is capped at 16, one GPU's share of a shared host) and with one thread.  Per
    linear: the weight is block-quantized untimed (once per optimizer step), then the timed part quantizes the
    sampled activation and gradient rows and runs the forward and DGrad GEMMs for `rows` token rows (all output
    columns) and WGrad for `rows` rows of dW over one 128-token group.  The one-thread run does the same for
    rows // 16 token rows (at least 1).  value = GEMM flops of the sample / time with all threads."""
    import numpy as np
    import oracle
    threads = oracle.default_threads()
    rows1 = max(1, rows // 16)
    flops = {threads: 0, 1: 0}
    elapsed = {threads: 0.0, 1: 0.0}
    for i, (name, K, N) in enumerate(wl.linears):
        h = workloads.host_linear(workloads.Workload(wl.name, 128, wl.linears, wl.outlier_frac, wl.seed, True, ""), i)
        wq, ws = oracle.quantize_blocks(h["w"], threads)
        for nt, r in ((threads, rows), (1, rows1)):
            t0 = time.perf_counter()
            xq, xs = oracle.quantize_rows(np.ascontiguousarray(h["x"][:r]), nt)
            dyq, dys = oracle.quantize_rows(np.ascontiguousarray(h["dy"][:r]), nt)
            oracle.gemm_fwd(xq, xs, wq, ws, mode=oracle.MFMA, threads=nt)
            oracle.gemm_dgrad(dyq, dys, wq, ws, mode=oracle.MFMA, threads=nt)
            dyqc, dysc = oracle.quantize_cols(np.ascontiguousarray(h["dy"][:, :r]), nt)
            xqc, xsc = oracle.quantize_cols(h["x"], nt)
            oracle.gemm_wgrad(dyqc, dysc, xqc, xsc, mode=oracle.MFMA, threads=nt)
            elapsed[nt] += time.perf_counter() - t0
            flops[nt] += 2 * r * N * K * 2 + 2 * r * K * 128
    host, aff = host_core_counts()
    return {"value": flops[threads] / elapsed[threads] / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "host_cores": host, "affinity_cores": aff,
            "value_1thread": flops[1] / elapsed[1] / 1e12,
            "sample": (f"per linear (weights block-quantized untimed): the sampled rows' 1x128 / 128x1 quantization, "
                       f"forward and dgrad for {rows} token rows, wgrad for {rows} rows of dW over one 128-token "
                       f"group; {flops[threads] / 1e9:.1f} GFLOP in {elapsed[threads]:.1f} s on {threads} threads. "
                       f"One thread: the same for {rows1} rows, {flops[1] / 1e9:.1f} GFLOP in {elapsed[1]:.1f} s"),
            "seconds": elapsed[threads] + elapsed[1]}


def producer_bytes(R, C, F):
    """Algorithmic bytes of the fused producers: RMSNorm reads x and the weight, writes codes, scales and rstd;
    SwiGLU reads gate and up, writes codes and scales."""
    return {"rmsnorm": R * C * 2 + C * 2 + R * C + (C // 128) * R * 4 + R * 4,
            "swiglu": R * 2 * F * 2 + R * F + (F // 128) * R * 4}


def producers_cpu_baseline(C, F, rows_rn, rows_sg, workloads):
    import oracle
    from oracle import producers
    oracle.lib()
    xb, wb = workloads.host_rmsnorm_inputs(21, rows_rn, C)
    gub = workloads.host_gate_up(22, rows_sg, F)
    t0 = time.perf_counter()
    producers.rmsnorm_quantize(xb, wb, 1e-5)
    t1 = time.perf_counter()
    producers.swiglu_quantize(gub)
    t2 = time.perf_counter()
    b = producer_bytes(rows_rn, C, F)["rmsnorm"] + producer_bytes(rows_sg, C, F)["swiglu"]
    return {"value": round(b / (t2 - t0) / 1e9, 4), "unit": "GB/s", "cores": oracle.default_threads(), "kind": "oracle",
            "sample": (f"oracle/producers.py: RMSNorm->1x128 of {rows_rn} rows x {C} ({t1 - t0:.1f} s, exact "
                       f"rational rstd) and SwiGLU->1x128 of {rows_sg} rows x {F} ({t2 - t1:.1f} s, numpy float64); "
                       "algorithmic bytes / time; the Python and numpy steps run on one core, the 1x128 quantizer "
                       "on the oracle's thread pool"),
            "seconds": round(t2 - t0, 2)}


PRODUCER_SOURCES = [os.path.join(ROOT, "fp8_precision_rl_amd", "csrc", f) for f in ("jetfp8_producers.hip", "jetfp8_common.h")]


def producer_traffic(workload, path=os.path.join(ROOT, "profiles", "producers_traffic.json")):
    """Per-launch HBM bytes of the producer kernels from rocprofv3 FETCH_SIZE / WRITE_SIZE (scaled by a 1 GiB
    copy), or None when the record is missing, was taken at another workload's shapes or on other kernel
    sources."""
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("workload") != workload or rec.get("source_sha256") != source_digest(PRODUCER_SOURCES):
        return None
    return {k: v["bytes"] for k, v in rec["kernels"].items()}


def timed_steps(torch, st, steps, step, with_events):
    """Time `steps` calls of step(c, ev) on stream st between two HIP events; ev collects per-launch event
    pairs when with_events.  Returns (ms per step, ev)."""
    ev = [] if with_events else None
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(st)
    for c in range(steps):
        step(c, ev)
    t1.record(st)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps, ev


def run_producers(args, torch, jf, workloads, wl):
    lin = {n: (K, N) for n, K, N in wl.linears}
    C, F, R = lin["qkv"][0], lin["down"][0], wl.M
    x, w = workloads.device_rmsnorm_inputs(31, R, C)
    gu = workloads.device_gate_up(32, R, F)
    u8, f32 = torch.uint8, torch.float32
    q_rn = torch.empty((R, C), dtype=u8, device=x.device)
    s_rn = torch.empty((C // 128, R), dtype=f32, device=x.device)
    r_rn = torch.empty((R,), dtype=f32, device=x.device)
    q_sg = torch.empty((R, F), dtype=u8, device=x.device)
    s_sg = torch.empty((F // 128, R), dtype=f32, device=x.device)
    st = torch.cuda.current_stream()
    byts = producer_bytes(R, C, F)

    def step(ev=None):
        for kind in ("rmsnorm", "swiglu", "rmsnorm"):           # attention norm, MLP activation, MLP norm
            a = b = None
            if ev is not None:
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(st)
            if kind == "rmsnorm":
                jf.jetfp8_rmsnorm_quantize(x, w, R, C, 1e-5, q_rn, s_rn, r_rn, None, st)
            else:
                jf.jetfp8_swiglu_quantize(gu, R, F, q_sg, s_sg, None, st)
            if ev is not None:
                b.record(st)
                ev.append((kind, a, b))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ms_step, _ = timed_steps(torch, st, args.steps, lambda c, ev: step(ev), with_events=False)
    ms_step_ev, ev = timed_steps(torch, st, args.steps, lambda c, ev: step(ev), with_events=True)
    per = {}
    for kind, a, b in ev:
        per.setdefault(kind, [0.0, 0])
        per[kind][0] += a.elapsed_time(b)
        per[kind][1] += 1
    total_bytes = 2 * byts["rmsnorm"] + byts["swiglu"]
    kern = {k: {"mean_launch_us": round(1e3 * v[0] / v[1], 2), "bytes_per_launch": byts[k],
                "achieved": round(byts[k] / (v[0] / v[1] * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(byts[k] / (v[0] / v[1] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)} for k, v in per.items()}
    traffic = producer_traffic(f"{wl.name} producers")
    for k in kern:
        kern[k]["traffic"] = traffic.get(k) if traffic else None
    dom = max(kern, key=lambda k: per[k][0])
    out = {
        "metric": "fused RMSNorm/SwiGLU -> 1x128 FP8 producers, algorithmic GB/s",
        "value": round(total_bytes / (ms_step * 1e-3) / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16 in, fp32/fp64 math, fp8_e4m3 out",
        "data": "synthetic (seeded torch generator on device: residual rows N(0,1) * 2^U(-4,4) with 1% outlier "
                "channels x50, norm weight 1+0.1N(0,1); gate 2N(0,1) with 1% outlier channels x20, up N(0,1))",
        "config": {"workload": f"{wl.name} producers", "tokens": R, "hidden": C, "ffn": F,
                   "step": "2 x RMSNorm->1x128 [tokens x hidden] + 1 x SwiGLU->1x128 [tokens x 2 ffn -> ffn]"},
        "roofline": dict(kern[dom], bound="hbm", kernel=f"{dom}_quant_kernel",
                         timing=f"HIP events around each launch, over {args.steps} more steps "
                                f"({ms_step_ev * 1e3:.1f} us per step with the events)"),
        "per_kernel": kern,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = producers_cpu_baseline(C, F, 2048, 6144, workloads)
    print(json.dumps(out), flush=True)


DECODE_COPIES = 3     # weight copies cycled by --decode: 3 x 218 MB of FP8 codes, beyond the 256 MB MALL


def decode_gemm_bytes(M, N, K):
    """Algorithmic bytes of one decode GEMM launch: FP8 weight codes and block scales, the activation codes and
    row scales, the bf16 output."""
    return N * K + (N // 128) * (K // 128) * 4 + M * K + (K // 128) * M * 4 + 2 * M * N


def decode_cpu_baseline(wl, M, workloads):
    """The oracle (unchanged) on the decode step itself, all four linears at M rows: 1x128 quantization of the
    activations and the forward GEMM (MFMA mode).  The weights are quantized by the oracle beforehand, outside
    the timed region, as the GPU path's are."""
    import oracle
    threads = oracle.default_threads()
    byts, elapsed = 0, 0.0
    for i, (name, K, N) in enumerate(wl.linears):
        h = workloads.host_linear(wl, i, M=M)
        wq, ws = oracle.quantize_blocks(h["w"], threads)
        t0 = time.perf_counter()
        xq, xs = oracle.quantize_rows(h["x"], threads)
        oracle.gemm_fwd(xq, xs, wq, ws, mode=oracle.MFMA, threads=threads)
        elapsed += time.perf_counter() - t0
        byts += decode_gemm_bytes(M, N, K) + (2 * M * K + M * K + (K // 128) * M * 4)
    return {"value": round(byts / elapsed / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"the whole decode step ({M} rows, four linears: activation quantization + forward GEMM) "
                      f"in {elapsed:.1f} s", "seconds": elapsed}


def decode_traffic(path=os.path.join(ROOT, "profiles", "decode_traffic.json")):
    """HBM bytes per decode GEMM launch recorded from rocprofv3 FETCH_SIZE / WRITE_SIZE runs of the 32-row decode
    workload, or None when absent or taken on a different kernel source."""
    try:
        tj = json.load(open(path))
    except (OSError, ValueError):
        return None
    if tj.get("kernel_source_sha256") != source_digest(DECODE_SOURCES):
        return None
    return tj.get("decode_bytes_per_launch")


def run_decode(args, torch, jf, workloads):
    wl = workloads.WORKLOADS["llama3_8b_decode_m32"]
    M = args.decode_rows or wl.M
    frag = not args.decode_rowmajor and M <= 64
    u8, f32, bf = torch.uint8, torch.float32, torch.bfloat16
    lin = []
    for i, (name, K, N) in enumerate(wl.linears):
        d = workloads.device_linear(wl, i, M=M)
        dev = d["x"].device
        copies = []
        for _ in range(DECODE_COPIES):
            wq = torch.empty((N, K), dtype=u8, device=dev)
            ws = torch.empty((N // 128, K // 128), dtype=f32, device=dev)
            jf.jetfp8_quantize(d["w"], N, K, jf.BLOCKS_128x128_FRAG if frag else jf.BLOCKS_128x128, wq, ws, None)
            copies.append((wq, ws))
        del d["w"]
        lin.append(dict(name=name, K=K, N=N, x=d["x"], copies=copies,
                        xq=torch.empty((M, K), dtype=u8, device=dev), xs=torch.empty((K // 128, M), dtype=f32, device=dev),
                        y=torch.empty((M, N), dtype=bf, device=dev)))
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()

    def step(c, ev=None):
        for L in lin:
            K, N = L["K"], L["N"]
            wq, ws = L["copies"][c % DECODE_COPIES]
            jf.jetfp8_quantize(L["x"], M, K, jf.ROWS_1x128, L["xq"], L["xs"], None, st)
            a = b = None
            if ev is not None:
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(st)
            (jf.jetfp8_gemm_fwd_frag if frag else jf.jetfp8_gemm_fwd)(L["xq"], L["xs"], wq, ws, L["y"], M, N, K, st)
            if ev is not None:
                b.record(st)
                ev.append((L["name"], decode_gemm_bytes(M, N, K), a, b))

    for c in range(args.warmup):
        step(c)
    torch.cuda.synchronize()
    # the step time comes from the timed steps run plainly; the per-launch durations from as many more steps with
    # a pair of HIP events around each GEMM (recording them costs the stream a few microseconds per launch); the
    # weight copies keep cycling from one region to the next
    nw, ns = args.warmup, args.steps
    ms_step, _ = timed_steps(torch, st, ns, lambda c, ev: step(nw + c, ev), with_events=False)
    ms_step_ev, ev = timed_steps(torch, st, ns, lambda c, ev: step(nw + ns + c, ev), with_events=True)
    step_bytes = sum(decode_gemm_bytes(M, L["N"], L["K"]) + 3 * M * L["K"] + (L["K"] // 128) * M * 4 for L in lin)
    gemm_ms = sum(a.elapsed_time(b) for _, _, a, b in ev)
    gemm_bytes = sum(n for _, n, _, _ in ev)
    per = {}
    for name, n, a, b in ev:
        per.setdefault(name, [0.0, 0, n])
        per[name][0] += a.elapsed_time(b)
        per[name][1] += 1
    rt = 1 if M <= 16 else (2 if M <= 32 else 4)
    out = {
        "metric": "rollout decode (FP8 activation quantize + forward GEMM over FP8 weights), algorithmic GB/s",
        "value": round(step_bytes / (ms_step * 1e-3) / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3 (fp32 accumulate, bf16 out)",
        "data": f"synthetic (seeded torch generator on device: X~N(0,1) with 0.1% outlier channels x50, "
                f"W~N(0,0.02^2)); {DECODE_COPIES} weight copies cycled past the 256 MB MALL",
        "config": {"workload": wl.name if M == wl.M else f"llama3_8b_decode_m{M}", "tokens": M,
                   "linears": [{"name": n, "K": K, "N": N} for n, K, N in wl.linears],
                   "step": "per linear: X rows quant (1x128), fwd GEMM against FP8 weights quantized beforehand",
                   "weights": "fragment order (jetfp8_gemm_fwd_frag)" if frag else "row-major (jetfp8_gemm_fwd)"},
        "roofline": {"bound": "hbm",
                     "kernel": (f"gemm_decode_wide_kernel<{rt}> (wide outputs), gemm_decode_split_kernel<{rt}, S> "
                                f"(narrow outputs), gemm_decode_roles_kernel<{rt}> (long contractions)"
                                if frag and rt <= 2 else f"gemm_decode_kernel<{rt}, {'true' if frag else 'false'}>"),
                     "achieved": round(gemm_bytes / (gemm_ms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gemm_bytes / (gemm_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": decode_traffic() if M == wl.M else None,
                     "launches": len(ev), "mean_launch_us": round(1e3 * gemm_ms / len(ev), 2),
                     "bytes_per_launch_mean": round(gemm_bytes / len(ev)),
                     "timing": f"HIP events around each launch, over {args.steps} more steps "
                               f"({ms_step_ev * 1e3:.1f} us per step with the events)"},
        "per_linear": {k: {"mean_launch_us": round(1e3 * v[0] / v[1], 2),
                           "gbs": round(v[2] / (v[0] / v[1] * 1e-3) / 1e9, 1)} for k, v in per.items()},
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on the decode step", file=sys.stderr, flush=True)
        out["cpu_baseline"] = decode_cpu_baseline(wl, M, workloads)
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path has no multi-GPU part.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import fp8_precision_rl_amd as jf
    import workloads

    jf.load_library()          # raises if the HIP library is not built: there is no fallback
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(3)
    wl = workloads.WORKLOADS[args.workload]
    if args.calibrate_copy:
        copy_calibration(torch)
    if args.producers:
        run_producers(args, torch, jf, workloads, wl)
        return
    if args.decode:
        run_decode(args, torch, jf, workloads)
        return
    layers = [Linear(wl, i, torch, workloads) for i in range(len(wl.linears))]
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    print(f"[bench] {wl.name}: {wl.description}; inputs resident", file=sys.stderr, flush=True)

    for _ in range(args.warmup):
        for L in layers:
            run_step(L, jf, st, fused=not args.separate_quant, x_from_fp8=args.x_from_fp8)
    torch.cuda.synchronize()
    print(f"[bench] warmup {args.warmup} done", file=sys.stderr, flush=True)

    ev = []
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    t_start.record()
    for _ in range(args.steps):
        for L in layers:
            run_step(L, jf, st, ev, fused=not args.separate_quant, x_from_fp8=args.x_from_fp8)
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    step_flops = sum(L.gemm_flops() for L in layers)
    value = step_flops / (ms_per_step * 1e-3) / 1e12

    gemm_ms = sum(a.elapsed_time(b) for k, _, _, a, b in ev if k == "gemm")
    gemm_flops = sum(f for k, _, f, _, _ in ev if k == "gemm")
    n_gemm = sum(1 for k, *_ in ev if k == "gemm")
    quant_ms = sum(a.elapsed_time(b) for k, _, _, a, b in ev if k == "quant")
    quant_bytes = sum(f for k, _, f, _, _ in ev if k == "quant")
    achieved = gemm_flops / (gemm_ms * 1e-3) / 1e12
    per = {}
    for k, name, amt, a, b in ev:
        key = f"{k}:{name}"
        per.setdefault(key, [0.0, 0.0])
        per[key][0] += a.elapsed_time(b)
        per[key][1] += amt
    traffic = recorded_traffic(args.traffic_json, wl.name)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 (fp32 accumulate, bf16 out)",
        "data": "synthetic (seeded torch generator on device: X~N(0,1) with 0.1% outlier channels x50, "
                "W~N(0,0.02^2), dY~1e-3*Student-t(3))",
        "config": {"workload": wl.name, "tokens": wl.M,
                   "linears": [{"name": n, "K": K, "N": N} for n, K, N in wl.linears],
                   "step": step_description(args)},
        "pct_of_fp8_peak": round(100 * value / FP8_PEAK_TFLOPS, 2),
        "gemm_only_tflops": round(achieved, 2),
        "wall_s": round(wall, 4),
        "roofline": {"bound": "mfma", "kernel": "gemm_pp_kernel (fwd, dgrad), gemm_large_kernel (wgrad, quarter-tile tails)", "achieved": round(achieved, 2),
                     "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / FP8_PEAK_TFLOPS, 4),
                     "traffic": traffic, "launches": n_gemm,
                     "mean_launch_us": round(1e3 * gemm_ms / max(n_gemm, 1), 2),
                     "flops_per_launch_mean": gemm_flops / max(n_gemm, 1)},
        "roofline_quant": {"bound": "hbm", "achieved": round(quant_bytes / (quant_ms * 1e-3) / 1e9, 1),
                           "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(quant_bytes / (quant_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "per_kernel": {k: {"ms_per_step": round(v[0] / args.steps, 4),
                           ("tflops" if k.startswith("gemm") else "gbs"):
                               round(v[1] / (v[0] * 1e-3) / (1e12 if k.startswith("gemm") else 1e9), 1)}
                       for k, v in per.items()},
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        rows = args.cpu_sample_rows or (64 if wl.M > 16384 else 128)
        out["cpu_baseline"] = cpu_baseline(wl, rows, workloads)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
