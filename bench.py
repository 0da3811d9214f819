#!/usr/bin/env python3
"""Benchmark of the quantized linear layer on one MI355X.

One step = the whole hot path on the large FP8 workload
(a BF16 [16384, 8192] ~ Student-t(3), b BF16 [8192, 8192] ~ N(0, 1/8192)):
per-tensor E4M3 quantize of a and of b (amax reduction, on-device step,
cast), then the scaled E4M3 GEMM 16384 x 8192 x 8192 with FP32 accumulation
and E4M3 output (out_scale = amax_prev / 448, amax_prev being the out_amax
of the previous step on the same inputs), which also publishes the step's
own out_amax.  The step is one ql_linear_forward call (the quantizes of a
and b share each pass's launch).  After the timed region the same work runs
again as its three C-ABI calls (ql_quantize, ql_quantize, ql_qgemm) with
HIP events between them on the stream they run on, which gives each
kernel's duration for the roofline and the quantize rates.

Prints one JSON line.  `value` is the step's GEMM work (2*M*N*K) divided by
the step time (inputs resident in HBM).  `roofline` is the GEMM kernel
against the dense FP8 matrix-core peak; `quantize` reports the quantize
calls against HBM peak; `cpu_baseline` is the oracle (plain C) timed on a
bounded sample of the same workload on this host's cores and scaled to the
full step.

`--copy-calibration` instead times a plain 1 GiB device copy (the known-size
kernel that scales the HBM byte counters of a profiler run) and exits.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "qgemm TFLOP/s & % dense FP8/INT8 MFMA peak; quantize GB/s & % HBM peak"
PEAK_FP8_TFLOPS = 5000.0        # MI355X dense FP8 matrix-core peak
PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E peak
# Profiler HBM byte counters of the GEMM kernel at this workload, per launch,
# already scaled by the copy calibration, with the hash of the kernel
# sources they were taken on; used only while the sources still match.
TRAFFIC_FILE = ROOT / "profiles" / "qgemm_nt_e4m3_large_fp8_traffic.json"
# The sources the pipelined E4M3 kernel is compiled from (the general and
# direct-to-LDS kernels in qgemm_impl.hpp / qgemm_dl.hpp, instantiated in the
# same unit, do not enter its code).
KERNEL_SOURCES = ["qgemm_nt.hpp", "qgemm_common.hpp", "qdev.hpp", "internal.hpp"]


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="time a plain 1 GiB device-to-device copy instead of the step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward timing")
    ap.add_argument("--cpu-rows", type=int, default=64, help="output rows in the oracle GEMM sample")
    ap.add_argument("--cpu-cols", type=int, default=4096, help="output columns in the oracle GEMM sample")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def time_events(fn, reps, torch):
    """Average milliseconds per call of fn over `reps` back-to-back calls,
    measured with events on torch's current stream (where fn launches)."""
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(reps):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / reps


def cpu_baseline(a_cpu, b_cpu, M, N, K, rows, cols):
    """Oracle timing on a bounded sample, scaled to one full step.

    Sample (roughly 10-30 s of host work): the per-tensor E4M3 quantize of
    the first 4096 rows of a and of b (one thread: the oracle quantize is a
    single call), and the exact GEMM of `rows` x `cols` outputs over the full
    K, split over the host's threads.  Step estimate = per-element quantize
    time x (M*K + N*K) + per-MAC GEMM time x M*N*K.
    """
    import numpy as np

    import oracle
    from precision_quantized_gemm_amd import synth

    threads = max(1, min(16, os.cpu_count() or 1))
    rows_q = 4096
    xa = synth.bf16_bits(a_cpu[:rows_q])
    xb = synth.bf16_bits(b_cpu[:rows_q])
    t0 = time.perf_counter()
    qa, sa, _ = oracle.quantize(xa, oracle.PER_TENSOR, oracle.E4M3)
    qb, sb, _ = oracle.quantize(xb, oracle.PER_TENSOR, oracle.E4M3)
    tq_wall = time.perf_counter() - t0
    tq = tq_wall / (2 * rows_q * K)
    ms = np.repeat(np.arange(rows), cols).astype(np.int64)
    ns = np.tile(np.arange(cols), rows).astype(np.int64)
    chunks = np.array_split(np.arange(ms.size), threads * 4)

    def work(idx):
        oracle.qgemm_entries(qa, 0, 0, qb, 0, 0, K, ms[idx], ns[idx], with_bound=False)

    t0 = time.perf_counter()
    with ThreadPoolExecutor(threads) as pool:
        list(pool.map(work, chunks))
    tg_wall = time.perf_counter() - t0
    tmac = tg_wall / (ms.size * K)
    step_s = tq * (M * K + N * K) + tmac * M * N * K
    return dict(value=2.0 * M * N * K / step_s / 1e12, unit="TFLOP/s", cores=threads, kind="oracle",
                sample=(f"quantize of the first {rows_q} rows of a and of b ({2 * rows_q * K} elements, "
                        f"1 thread, {tq_wall:.1f} s) and the exact GEMM of {rows}x{cols} outputs x K={K} "
                        f"({ms.size * K} MACs, {threads} threads, {tg_wall:.1f} s); scaled to the full "
                        f"{M}x{N}x{K} step"),
                step_seconds_estimate=step_s)


def time_backward(torch, q, synth, dev, reps):
    """ms per ql_linear_backward call on the MLP-up layer's backward and the
    rate of its two products (2 x 2*M*N*K flops)."""
    d = synth.workload("mlp_backward")
    g = d["g"].to(dev)
    fx = q.quantize(d["x"].to(dev), "per_tensor", "e4m3")
    fw = q.quantize(d["w"].to(dev), "per_tensor", "e4m3")
    ws = q.new_workspace(dev)
    run = lambda: q.linear_backward(g, fx[0], fx[1], fw[0], fw[1], ws=ws)
    for _ in range(3):
        run()
    ms = time_events(run, reps, torch)
    M, N = g.shape
    K = fx[0].shape[1]
    flops = 2 * 2.0 * M * N * K
    return {"workload": f"g BF16 [{M},{N}] N(0,1e-3) -> E5M2; x_q [{M},{K}], w_q [{N},{K}] E4M3; dX, dW (BF16), "
                        "grad_bias in one ql_linear_backward",
            "ms_per_call": round(ms, 5), "gemm_TFLOPs": round(flops / (ms * 1e-3) / 1e12, 2),
            "frac_fp8_peak": round(flops / (ms * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4)}


def time_per_head(torch, q, _lib, synth, dev, reps):
    """The per-head attention products of the per-head workload (BH = 16,
    N = 196, D = 64): per-head E4M3 quantize of q, k, p, v
    (ql_quantize_groups), S = Q.K^T and O = P.V with N != M (V MN-major) as
    ql_qgemm_batched with one scale per head on both operands."""
    d = {k: v.to(dev) for k, v in synth.workload("per_head").items()}
    BH, N, D = d["q"].shape
    NK = d["v"].shape[1]
    f = {}

    def quant_all():
        for role, g in (("q", N), ("k", N), ("p", N), ("v", NK)):
            f[role] = q.quantize_groups(d[role], g, "e4m3")

    quant_all()
    s_out = torch.empty((BH, N, N), dtype=torch.bfloat16, device=dev)
    o_out = torch.empty((BH, N, D), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream().cuda_stream

    def qk():
        (aq, sa, _), (bq, sb, _) = f["q"], f["k"]
        q.ql_qgemm_batched(aq.data_ptr(), _lib.QL_FMT_E4M3, _lib.QL_K_MAJOR, D, N * D,
                           bq.data_ptr(), _lib.QL_FMT_E4M3, _lib.QL_K_MAJOR, D, N * D, BH, N, N, D,
                           sa.data_ptr(), N, sb.data_ptr(), N, None, 0, s_out.data_ptr(), _lib.QL_DT_BF16, N, N * N,
                           None, None, None, stream)

    def pv():
        (aq, sa, _), (vq, sv, _) = f["p"], f["v"]
        q.ql_qgemm_batched(aq.data_ptr(), _lib.QL_FMT_E4M3, _lib.QL_K_MAJOR, NK, N * NK,
                           vq.data_ptr(), _lib.QL_FMT_E4M3, _lib.QL_MN_MAJOR, D, NK * D, BH, N, D, NK,
                           sa.data_ptr(), N, sv.data_ptr(), D, None, 0, o_out.data_ptr(), _lib.QL_DT_BF16, D, N * D,
                           None, None, None, stream)

    for _ in range(3):
        quant_all(); qk(); pv()
    ms_q = time_events(quant_all, reps, torch)
    ms_qk = time_events(qk, reps, torch)
    ms_pv = time_events(pv, reps, torch)
    fl_qk, fl_pv = 2.0 * BH * N * N * D, 2.0 * BH * N * D * NK
    return {"workload": f"per-head q,k [{BH},{N},{D}], p [{BH},{N},{NK}], v [{BH},{NK},{D}] FP32 -> E4M3 "
                        "per head; S = Q.K^T, O = P.V (BF16 out)",
            "quantize_4_tensors_ms": round(ms_q, 5), "qk_ms": round(ms_qk, 5), "pv_ms": round(ms_pv, 5),
            "qk_TFLOPs": round(fl_qk / (ms_qk * 1e-3) / 1e12, 2), "pv_TFLOPs": round(fl_pv / (ms_pv * 1e-3) / 1e12, 2),
            "note": "launch-bound sizes (tens of MFLOP per product)"}


SCLK_FILES = sorted(Path("/sys/class/drm").glob("card*/device/pp_dpm_sclk")) if Path("/sys/class/drm").exists() else []


def read_sclk_mhz():
    """The current shader clock (the level marked '*' in pp_dpm_sclk), or
    None where the file is not readable."""
    for f in SCLK_FILES:
        try:
            for line in f.read_text().splitlines():
                if line.rstrip().endswith("*"):
                    return float(line.split(":")[1].strip().split("Mhz")[0].split("MHz")[0])
        except (OSError, ValueError, IndexError):
            continue
    return None


def sclk_under(fn, torch, launches):
    """Average shader clock (MHz) sampled every 2 ms while `launches` calls
    of fn run back to back on the GPU (all enqueued first), or None."""
    if read_sclk_mhz() is None:
        return None
    torch.cuda.synchronize()
    done = torch.cuda.Event()
    for _ in range(launches):
        fn()
    done.record()
    samples = []
    while not done.query():
        v = read_sclk_mhz()
        if v is not None:
            samples.append(v)
        time.sleep(0.002)
    torch.cuda.synchronize()
    # Drop the first and last tenth (ramp and drain).
    k = len(samples) // 10
    core = samples[k:len(samples) - k] if len(samples) > 10 else samples
    return round(sum(core) / len(core), 1) if core else None


def time_configs(torch, q, _lib, synth, dev, reps):
    """The small configurations of the method on the same library calls:
    the tiny linear layer (linear_forward, x [512,128], W [128,128]), per-row
    INT8 (quantize a [128,1024] and b [512,1024] per row, INT8 GEMM, FP32
    out = acc * sa[m] * sb[n]) and the MLP-up layer (linear_forward, x
    [2048,1024], W [4096,1024]).  Each step is timed eagerly and as a
    replayed HIP graph of the same calls (no host launch cost); the graph's
    result is checked against the eager one."""
    P = lambda t: None if t is None else t.data_ptr()
    f1 = lambda: torch.empty(1, dtype=torch.float32, device=dev)
    ws = q.new_workspace(dev)
    stream = lambda: torch.cuda.current_stream().cuda_stream
    out = {}

    def linear(name, x, w, bias):
        M, K = x.shape
        N = w.shape[0]
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        xq = torch.empty((M, K), dtype=torch.uint8, device=dev)
        wq = torch.empty((N, K), dtype=torch.uint8, device=dev)
        sx, ax, sw, aw = f1(), f1(), f1(), f1()
        run = lambda: q.ql_linear_forward(P(x), _lib.QL_DT_BF16, M, K, P(w), N, P(bias), _lib.QL_DT_FP32,
                                          _lib.QL_FMT_E4M3, None, None, P(y), _lib.QL_DT_BF16, None, None,
                                          P(xq), P(sx), P(ax), P(wq), P(sw), P(aw), P(ws), stream())
        return run, y, 2.0 * M * N * K

    def rowwise(a, b):
        M, K = a.shape
        N = b.shape[0]
        aq = torch.empty((M, K), dtype=torch.uint8, device=dev)
        bq = torch.empty((N, K), dtype=torch.uint8, device=dev)
        sa, am = torch.empty(M, device=dev), torch.empty(M, device=dev)
        sb, bm = torch.empty(N, device=dev), torch.empty(N, device=dev)
        y = torch.empty((M, N), dtype=torch.float32, device=dev)

        def run():
            q.ql_quantize(P(a), _lib.QL_DT_FP32, M, K, K, _lib.QL_PER_ROW, _lib.QL_FMT_INT8, None, P(aq), K, P(sa),
                          P(am), None, stream())
            q.ql_quantize(P(b), _lib.QL_DT_FP32, N, K, K, _lib.QL_PER_ROW, _lib.QL_FMT_INT8, None, P(bq), K, P(sb),
                          P(bm), None, stream())
            q.ql_qgemm(P(aq), _lib.QL_FMT_INT8, _lib.QL_K_MAJOR, K, P(bq), _lib.QL_FMT_INT8, _lib.QL_K_MAJOR, K,
                       M, N, K, P(sa), _lib.QL_PER_ROW, P(sb), _lib.QL_PER_ROW, None, 0, P(y), _lib.QL_DT_FP32, N,
                       None, None, P(ws), stream())
        return run, y, 2.0 * M * N * K

    t1 = synth.workload("tiny_linear")
    t2 = synth.workload("rowwise_int8")
    t3 = synth.workload("mlp_up")
    cases = {
        "tiny_linear": linear("tiny_linear", t1["x"].to(dev), t1["w"].to(dev), t1["bias"].to(dev)),
        "rowwise_int8": rowwise(t2["a"].to(dev), t2["b"].to(dev)),
        "mlp_up": linear("mlp_up", t3["x"].to(dev), t3["w"].to(dev), t3["bias"].to(dev)),
    }
    for name, (run, y, flops) in cases.items():
        for _ in range(3):
            run()
        ms_eager = time_events(run, reps, torch)
        torch.cuda.synchronize()
        ref = y.clone()
        entry = {"ms_eager": round(ms_eager, 5), "TFLOPs_eager": round(flops / (ms_eager * 1e-3) / 1e12, 2)}
        out[name] = entry
        try:
            entry.update(graph_replay(run, y, ref, flops, torch, reps))
        except RuntimeError as e:                  # report, keep the benchmark line
            entry["graph_error"] = str(e)[:200]
    return out


def graph_replay(run, y, ref, flops, torch, reps):
    """Capture run() once in a HIP graph, replay it `reps` times; the result
    must equal the eager one after every timing."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()                                   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run()
    g.replay()
    torch.cuda.synchronize()
    same = bool(torch.equal(y, ref))
    ms_graph = time_events(g.replay, reps, torch)
    torch.cuda.synchronize()
    same = same and bool(torch.equal(y, ref))
    return {"ms_graph_replay": round(ms_graph, 5), "TFLOPs_graph": round(flops / (ms_graph * 1e-3) / 1e12, 2),
            "graph_matches_eager": same}


def time_int8_large(torch, q, _lib, dev, M, N, K, reps):
    """INT8 GEMM at the benchmark shape (an extra, clearly INT8: random codes
    in [-127, 127], per-row scales, raw INT32 accumulator output), on the
    general kernel."""
    g = torch.Generator(device=dev)
    g.manual_seed(0x5EED0008)
    a = torch.randint(-127, 128, (M, K), device=dev, dtype=torch.int32, generator=g).to(torch.int8)
    b = torch.randint(-127, 128, (N, K), device=dev, dtype=torch.int32, generator=g).to(torch.int8)
    s1 = torch.ones(max(M, N), device=dev)
    out = torch.empty((M, N), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    run = lambda: q.ql_qgemm(a.data_ptr(), _lib.QL_FMT_INT8, _lib.QL_K_MAJOR, K, b.data_ptr(), _lib.QL_FMT_INT8,
                             _lib.QL_K_MAJOR, K, M, N, K, s1.data_ptr(), _lib.QL_PER_ROW, s1.data_ptr(),
                             _lib.QL_PER_ROW, None, 0, out.data_ptr(), _lib.QL_DT_INT32, N, None, None, None, stream)
    for _ in range(2):
        run()
    ms = time_events(run, reps, torch)
    ops = 2.0 * M * N * K
    del a, b, out
    return {"workload": f"INT8 {M}x{N}x{K}, per-row scales, INT32 out", "ms_per_launch": round(ms, 5),
            "TOPs": round(ops / (ms * 1e-3) / 1e12, 1), "frac_int8_peak": round(ops / (ms * 1e-3) / 1e12 / 5000.0, 4)}


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        h.update((ROOT / "precision_quantized_gemm_amd" / "csrc" / name).read_bytes())
    return h.hexdigest()[:16]


def gemm_traffic():
    """HBM bytes per GEMM launch from the committed counter summary, or None
    when the kernel sources changed since it was taken."""
    if not TRAFFIC_FILE.exists():
        return None
    t = json.loads(TRAFFIC_FILE.read_text())
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t["hbm_bytes_per_launch"]


def copy_calibration(torch, dev, nbytes=1 << 30, reps=10):
    """A plain device copy of known size: every launch reads and writes
    exactly `nbytes` of HBM, so a profiler's fetch / write byte counters on
    it give the factor between those counters and real bytes."""
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        dst.copy_(src)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "ms_per_copy": round(ms, 5),
                      "GBps_read_plus_write": round(2 * nbytes / (ms * 1e-3) / 1e9, 1), "launches": reps + 1}),
          flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import precision_quantized_gemm_amd as q
    from precision_quantized_gemm_amd import _lib, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        copy_calibration(torch, dev)
        return
    log("generating inputs")
    d = synth.workload("large_fp8")
    a_cpu, b_cpu = d["a"], d["b"]
    M, K = a_cpu.shape
    N = b_cpu.shape[0]
    a = a_cpu.to(dev)
    b = b_cpu.to(dev)
    u8 = torch.uint8
    out = torch.empty((M, N), dtype=u8, device=dev)
    x_q = torch.empty((M, K), dtype=u8, device=dev)
    w_q = torch.empty((N, K), dtype=u8, device=dev)
    f1 = lambda: torch.empty(1, dtype=torch.float32, device=dev)
    sx, amax_x, sw, amax_w, out_amax = f1(), f1(), f1(), f1(), f1()
    out_scale = torch.ones(1, dtype=torch.float32, device=dev)
    ws = q.new_workspace(dev)
    stream = torch.cuda.current_stream().cuda_stream
    P = lambda t: t.data_ptr()

    def quant(x, rows, xq, s, am):
        return lambda: q.ql_quantize(P(x), _lib.QL_DT_BF16, rows, K, K, 0, 0, None, P(xq), K, P(s), P(am),
                                     P(ws), stream)

    qa, qb = quant(a, M, x_q, sx, amax_x), quant(b, N, w_q, sw, amax_w)

    def gemm():
        q.ql_qgemm(P(x_q), 0, 0, K, P(w_q), 0, 0, K, M, N, K, P(sx), 0, P(sw), 0, None, 0,
                   P(out), _lib.QL_DT_E4M3, N, P(out_scale), P(out_amax), P(ws), stream)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        qa()
        if ev is not None:
            ev[1].record()
        qb()
        if ev is not None:
            ev[2].record()
        gemm()
        if ev is not None:
            ev[3].record()

    # The step: one ql_linear_forward call (quantize a and b per tensor, the
    # quantizes sharing each pass's launch, then the GEMM with E4M3 output
    # and out_amax).
    def fused_step():
        q.ql_linear_forward(P(a), _lib.QL_DT_BF16, M, K, P(b), N, None, 0, _lib.QL_FMT_E4M3, None, None,
                            P(out), _lib.QL_DT_E4M3, P(out_scale), P(out_amax), P(x_q), P(sx), P(amax_x),
                            P(w_q), P(sw), P(amax_w), P(ws), stream)

    log("warmup")
    fused_step()
    torch.cuda.synchronize()
    out_scale.copy_(out_amax / 448.0)           # amax_prev / 448
    for _ in range(max(0, args.warmup - 1)):
        fused_step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    e_start, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    e_start.record()
    for _ in range(args.steps):
        fused_step()
    e_end.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0
    ms_step = e_start.elapsed_time(e_end) / args.steps

    # Breakdown (after the timed region): the same work as three calls with
    # events between them, for the per-kernel rates and the roofline.
    log("per-call breakdown")
    for _ in range(2):
        step()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for ev in events:
        step(ev)
    torch.cuda.synchronize()
    ms_step_calls = events[0][0].elapsed_time(events[-1][3]) / args.steps
    ms_qa = sum(ev[0].elapsed_time(ev[1]) for ev in events) / args.steps
    ms_qb = sum(ev[1].elapsed_time(ev[2]) for ev in events) / args.steps
    ms_gemm = sum(ev[2].elapsed_time(ev[3]) for ev in events) / args.steps
    gemm_each = sorted(ev[2].elapsed_time(ev[3]) for ev in events)
    pct = lambda f: gemm_each[min(len(gemm_each) - 1, int(f * len(gemm_each)))]
    flops = 2.0 * M * N * K
    value = flops / (ms_step * 1e-3) / 1e12
    gemm_tflops = flops / (ms_gemm * 1e-3) / 1e12
    # Quantize bytes per BF16 element, per-tensor current scaling: the
    # method reads x twice (amax pass, cast pass) and writes one code byte:
    # 5 B; the compulsory traffic is 3 B.
    qa_bytes5, qa_bytes3 = 5.0 * M * K, 3.0 * M * K
    qb_bytes5 = 5.0 * N * K
    qa_gbps = qa_bytes5 / (ms_qa * 1e-3) / 1e9
    qb_gbps = qb_bytes5 / (ms_qb * 1e-3) / 1e9

    # Single-pass delayed scaling through an amax history ring on the same
    # a (one read of BF16 x, one code byte written: 3 B/elem), timed on its
    # own after the step.
    ring = torch.zeros(17, dtype=torch.float32, device=dev)
    ring[-1] = 1.0
    su, am = f1(), f1()
    ring_idx = [0]

    def qa_ring():
        q.ql_quantize_ring(P(a), _lib.QL_DT_BF16, M, K, K, _lib.QL_FMT_E4M3, P(ring), 16, ring_idx[0] % 16, 0,
                           P(x_q), K, P(su), P(am), P(ws), stream)
        ring_idx[0] += 1

    for _ in range(3):
        qa_ring()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        qa_ring()
    e1.record()
    torch.cuda.synchronize()
    ms_ring = e0.elapsed_time(e1) / args.steps

    # Static FP8 inference on the same layer: w arrives quantized (the w_q /
    # sw the step produced), so a call quantizes a and runs the GEMM.
    def static_step():
        q.ql_linear_forward_static(P(a), _lib.QL_DT_BF16, M, K, P(w_q), N, P(sw), None, 0, None,
                                   _lib.QL_FMT_E4M3, None, P(out), _lib.QL_DT_E4M3, P(out_scale), P(out_amax),
                                   P(x_q), P(sx), P(amax_x), P(ws), stream)

    for _ in range(3):
        static_step()
    ms_static = time_events(static_step, args.steps, torch)



    # Backward of the MLP-up layer (G [2048, 4096] BF16 -> E5M2, x_q
    # [2048, 1024] and w_q [4096, 1024] E4M3): one ql_linear_backward call
    # (quantize G, dX = G.W, dW = G^T.X with MN-major operands, grad_bias).
    bwd = None
    if not args.no_backward:
        log("backward")
        bwd = time_backward(torch, q, synth, dev, args.steps)

    log("per-head batched products")
    per_head = time_per_head(torch, q, _lib, synth, dev, args.steps)

    log("small configurations")
    small = time_configs(torch, q, _lib, synth, dev, args.steps)

    log("INT8 at the benchmark shape")
    int8 = time_int8_large(torch, q, _lib, dev, M, N, K, 10)

    log("shader clock under the GEMM")
    sclk = sclk_under(gemm, torch, 500)

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(a_cpu, b_cpu, M, N, K, args.cpu_rows, args.cpu_cols)

    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {
            "workload": "large_fp8: quantize a[16384,8192] bf16 Student-t(3) and b[8192,8192] bf16 N(0,1/8192) "
                        "per-tensor E4M3, then E4M3 GEMM 16384x8192x8192 FP32-acc, E4M3 out "
                        "(out_scale = amax_prev/448); per step one ql_linear_forward (quantize a and b, the GEMM)",
            "M": M, "N": N, "K": K, "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(gemm_tflops, 2),
            "peak": PEAK_FP8_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(gemm_tflops / PEAK_FP8_TFLOPS, 4),
            "traffic": gemm_traffic(),
            "kernel": "qgemm_nt_kernel<E4M3,E4M3> (256x256x128 tiles)",
            "ms_per_launch": round(ms_gemm, 5),
            "ms_per_launch_p10_p50_p90": [round(pct(0.1), 5), round(pct(0.5), 5), round(pct(0.9), 5)],
            "sclk_mhz_under_gemm": sclk,
            "frac_at_measured_sclk": None if not sclk else round(gemm_tflops / (PEAK_FP8_TFLOPS * sclk / 2400.0), 4),
            "per_launch_flops": flops,
        },
        "quantize": {
            "a_ms": round(ms_qa, 5), "b_ms": round(ms_qb, 5),
            "bytes_per_elem": "5 (two reads of BF16 x, one code byte written)",
            "a_GBps_5B_per_elem": round(qa_gbps, 1),
            "a_GBps_3B_per_elem": round(qa_bytes3 / (ms_qa * 1e-3) / 1e9, 1),
            "b_GBps_5B_per_elem": round(qb_gbps, 1),
            "a_frac_hbm_peak_5B": round(qa_gbps / PEAK_HBM_GBPS, 4),
            "a_ring_ms": round(ms_ring, 5),
            "a_ring_GBps_3B_per_elem": round(qa_bytes3 / (ms_ring * 1e-3) / 1e9, 1),
            "a_ring_frac_hbm_peak": round(qa_bytes3 / (ms_ring * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
            "a_ring_note": "ql_quantize_ring (delayed scaling, 16-entry history), back to back on a",
            "peak_GBps": PEAK_HBM_GBPS,
        },
        "step_as_three_calls": {"ms_per_step": round(ms_step_calls, 5),
                                "TFLOPs": round(flops / (ms_step_calls * 1e-3) / 1e12, 2),
                                "workload": "the same step as ql_quantize(a), ql_quantize(b), ql_qgemm with events between"},
        "static_inference": {"ms_per_step": round(ms_static, 5),
                             "TFLOPs": round(flops / (ms_static * 1e-3) / 1e12, 2),
                             "workload": "ql_linear_forward_static: quantize a, GEMM with the pre-quantized b"},
        "linear_backward": bwd,
        "per_head": per_head,
        "small_configs": small,
        "int8_large": int8,
        "cpu_baseline": None if cpu is None else {k: (round(v, 6) if isinstance(v, float) else v)
                                                 for k, v in cpu.items()},
        "wall_s_timed_region": round(t_wall, 4),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
