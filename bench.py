#!/usr/bin/env python3
"""Benchmark of the quantized linear layer on one MI355X.

One step = the whole hot path on the large FP8 workload
(a BF16 [16384, 8192] ~ Student-t(3), b BF16 [8192, 8192] ~ N(0, 1/8192)):
per-tensor E4M3 quantize of a and of b (amax reduction, on-device step,
cast), then the scaled E4M3 GEMM 16384 x 8192 x 8192 with FP32 accumulation
and E4M3 output (out_scale = amax_prev / 448, amax_prev being the out_amax
of the previous step on the same inputs), which also publishes the step's
own out_amax.  The step is one ql_linear_forward call (the quantizes of a
and b share each pass's launch); consecutive steps alternate between two
copies of the inputs, so no step finds its inputs in the memory-side
cache.  After W warm-up steps, further untimed steps run until 0.5 s of
warm-up have passed; then K steps are timed, with an event after each for
the per-step p10 / p50 / p90.

After the timed region the same work runs again as its three C-ABI calls
(ql_quantize, ql_quantize, ql_qgemm) with HIP events between them on the
stream they run on, which gives the GEMM's duration for the roofline.  The
quantize rates are timed on rotated copies of a and b (768 / 640 MiB) next
to the memory system's ceiling for the same access pattern
(ql_stream_probe).

Prints one JSON line.  `value` is the step's GEMM work (2*M*N*K) divided by
the step time (inputs resident in HBM).  `roofline` is the GEMM kernel
against the dense FP8 matrix-core peak; `quantize` reports the quantize
calls against HBM peak and the measured ceiling; `cpu_baseline` is the
oracle (plain C) timed on a bounded sample of the same workload over this
host's cores and scaled to the full step; `cpu_baseline_configs` times the
oracle on the small configurations next to their GPU times.

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
    ap.add_argument("--cpu-rows", type=int, default=32, help="full output rows in the oracle GEMM sample")
    ap.add_argument("--cpu-full", action="store_true",
                    help="run the oracle GEMMs of the MLP-up and backward configurations in full (minutes)")
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


def host_threads():
    """Threads for the oracle legs: the CPUs this process may run on,
    capped by OMP_NUM_THREADS when the environment sets it (the host's
    share of cores for this GPU)."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    cap = os.environ.get("OMP_NUM_THREADS")
    if cap and cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def oracle_quantize_threaded(oracle, x_bits, gran, fmt, pool, threads):
    """The oracle's quantize of x split over row chunks: per tensor, the
    amax of every chunk (oracle.amax_raw), then every chunk's cast with the
    whole tensor's step (oracle.quantize with that step given); per row,
    each chunk on its own.  Returns the codes."""
    import numpy as np
    chunks = [c for c in np.array_split(np.arange(x_bits.shape[0]), threads * 2) if c.size]
    if gran == oracle.PER_ROW:
        parts = list(pool.map(lambda c: oracle.quantize(x_bits[c], gran, fmt)[0], chunks))
        return np.concatenate(parts)
    amax = max(pool.map(lambda c: float(oracle.amax_raw(x_bits[c], oracle.PER_TENSOR)[0]), chunks))
    floor = float(oracle.amax_floor(fmt))
    step = np.float32(max(np.float32(amax), np.float32(floor))) / np.float32(oracle.qmax(fmt))
    parts = list(pool.map(lambda c: oracle.quantize(x_bits[c], oracle.PER_TENSOR, fmt,
                                                     scale_in=np.array([step], np.float32))[0], chunks))
    return np.concatenate(parts)


def oracle_gemm_seconds(oracle, pool, threads, a, af, al, b, bf, bl, K, M, N, rows):
    """Wall time of the oracle's exact GEMM over `rows` output rows (all N
    columns), the entries split over the threads, and the factor M / rows
    that scales it to the whole product."""
    import numpy as np
    rows = min(rows, M)
    ms = np.repeat(np.arange(rows), N).astype(np.int64)
    ns = np.tile(np.arange(N), rows).astype(np.int64)
    parts = np.array_split(np.arange(ms.size), threads * 4)
    t0 = time.perf_counter()
    list(pool.map(lambda i: oracle.qgemm_entries(a, af, al, b, bf, bl, K, ms[i], ns[i], with_bound=False), parts))
    return time.perf_counter() - t0, M / rows


def cpu_baseline(a_cpu, b_cpu, M, N, K, rows, threads):
    """Oracle timing for the benchmark step, on a bounded sample.

    Sample (roughly 10-30 s of host work): the per-tensor E4M3 quantize of
    all of a and b (amax of every row chunk, then every chunk's cast with
    the tensor's step, over `threads` threads), and the exact GEMM of
    `rows` full output rows (rows x N entries over the full K), over the
    same threads.  Step estimate = quantize time + GEMM time x M / rows.
    """
    import oracle
    from precision_quantized_gemm_amd import synth

    with ThreadPoolExecutor(threads) as pool:
        xa, xb = synth.bf16_bits(a_cpu), synth.bf16_bits(b_cpu)
        t0 = time.perf_counter()
        qa = oracle_quantize_threaded(oracle, xa, oracle.PER_TENSOR, oracle.E4M3, pool, threads)
        qb = oracle_quantize_threaded(oracle, xb, oracle.PER_TENSOR, oracle.E4M3, pool, threads)
        tq = time.perf_counter() - t0
        tg, scale = oracle_gemm_seconds(oracle, pool, threads, qa, 0, 0, qb, 0, 0, K, M, N, rows)
    step_s = tq + tg * scale
    return dict(value=2.0 * M * N * K / step_s / 1e12, unit="TFLOP/s", cores=threads, kind="oracle",
                sample=(f"quantize of all of a and b ({M * K + N * K} elements, {tq:.1f} s) and the exact GEMM "
                        f"of {rows} full output rows ({rows}x{N} entries x K={K}, {tg:.1f} s, scaled x{scale:g} "
                        f"to {M} rows), each over {threads} threads; estimate of the whole "
                        f"{M}x{N}x{K} step"),
                step_seconds_estimate=step_s,
                host_cpus_visible=os.cpu_count(),
                host_cpus_usable=len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None)


def oracle_configs(threads, full):
    """The oracle on the small configurations (seconds per step, the same
    work as the GPU lines they sit next to).  C1 and C2 run in full; C3's
    and C4's GEMMs run in full with `full`, else on row slabs scaled to the
    whole product (labelled)."""
    import numpy as np

    import oracle
    from precision_quantized_gemm_amd import synth

    out = {}
    with ThreadPoolExecutor(threads) as pool:
        def leg(name, quantize, gemms):
            t0 = time.perf_counter()
            codes = quantize()
            tq = time.perf_counter() - t0
            tg, notes = 0.0, []
            for g in gemms:
                t, f = g(codes)
                tg += t * f
                notes.append("full" if f == 1 else f"{t:.2f} s slab x{f:g}")
            out[name] = {"oracle_s": round(tq + tg, 4), "quantize_s": round(tq, 4), "gemm_s": round(tg, 4),
                         "gemm": ", ".join(notes)}

        d = synth.workload("tiny_linear")
        bits = lambda t: synth.bf16_bits(t)
        leg("tiny_linear",
            lambda: [oracle_quantize_threaded(oracle, bits(d["x"]), 0, 0, pool, threads),
                     oracle_quantize_threaded(oracle, bits(d["w"]), 0, 0, pool, threads)],
            [lambda c: oracle_gemm_seconds(oracle, pool, threads, c[0], 0, 0, c[1], 0, 0, 128, 512, 128, 512)])
        d2 = synth.workload("rowwise_int8")
        leg("rowwise_int8",
            lambda: [oracle_quantize_threaded(oracle, d2["a"].numpy(), 1, 2, pool, threads),
                     oracle_quantize_threaded(oracle, d2["b"].numpy(), 1, 2, pool, threads)],
            [lambda c: oracle_gemm_seconds(oracle, pool, threads, c[0], 2, 0, c[1], 2, 0, 1024, 128, 512, 128)])
        d3 = synth.workload("mlp_up")
        leg("mlp_up",
            lambda: [oracle_quantize_threaded(oracle, bits(d3["x"]), 0, 0, pool, threads),
                     oracle_quantize_threaded(oracle, bits(d3["w"]), 0, 0, pool, threads)],
            [lambda c: oracle_gemm_seconds(oracle, pool, threads, c[0], 0, 0, c[1], 0, 0, 1024, 2048, 4096,
                                           2048 if full else 16)])
        d4 = synth.workload("mlp_backward")
        xq = oracle_quantize_threaded(oracle, bits(d4["x"]), 0, 0, pool, threads)
        wq = oracle_quantize_threaded(oracle, bits(d4["w"]), 0, 0, pool, threads)
        # dX [2048, 1024] = g [2048, 4096] . W (W read MN-major); dW [4096, 1024]
        # = g^T . X (both MN-major); the column sums of g for grad_bias.
        leg("mlp_backward",
            lambda: [oracle_quantize_threaded(oracle, bits(d4["g"]), 0, 1, pool, threads)],
            [lambda c: oracle_gemm_seconds(oracle, pool, threads, c[0], 1, 0, wq, 0, 1, 4096, 2048, 1024,
                                           2048 if full else 8),
             lambda c: oracle_gemm_seconds(oracle, pool, threads, c[0], 1, 1, xq, 0, 1, 2048, 4096, 1024,
                                           4096 if full else 16)])
    return out


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


def time_mlp_products(torch, q, _lib, synth, dev, reps):
    """Each product of the MLP-up layer alone (ql_qgemm, BF16 out): the
    forward x_q . w_q^T + bias (2048 x 4096 x 1024, both K-major), dX =
    g_q . W (2048 x 1024 x 4096, W read MN-major) and dW = g_q^T . X
    (4096 x 1024 x 2048, both read MN-major)."""
    d = synth.workload("mlp_backward")
    up = synth.workload("mlp_up")
    P = lambda t: t.data_ptr()
    fx = q.quantize(up["x"].to(dev), "per_tensor", "e4m3")
    fw = q.quantize(up["w"].to(dev), "per_tensor", "e4m3")
    fg = q.quantize(d["g"].to(dev), "per_tensor", "e5m2")
    bias = up["bias"].to(dev)
    (xq, sx, _), (wq, sw, _), (gq, sg, _) = fx, fw, fg
    M, K = xq.shape
    N = wq.shape[0]
    stream = torch.cuda.current_stream().cuda_stream
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    dw = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    E4, E5, KM, MN, BF = _lib.QL_FMT_E4M3, _lib.QL_FMT_E5M2, _lib.QL_K_MAJOR, _lib.QL_MN_MAJOR, _lib.QL_DT_BF16
    ws = P(q.new_workspace(dev))
    runs = {
        "forward": (lambda: q.ql_qgemm(P(xq), E4, KM, K, P(wq), E4, KM, K, M, N, K, P(sx), 0, P(sw), 0, P(bias),
                                       _lib.QL_DT_FP32, P(y), BF, N, None, None, ws, stream), (M, N, K)),
        "dX": (lambda: q.ql_qgemm(P(gq), E5, KM, N, P(wq), E4, MN, K, M, K, N, P(sg), 0, P(sw), 0, None, 0,
                                  P(dx), BF, K, None, None, ws, stream), (M, K, N)),
        "dW": (lambda: q.ql_qgemm(P(gq), E5, MN, N, P(xq), E4, MN, K, N, K, M, P(sg), 0, P(sx), 0, None, 0,
                                  P(dw), BF, K, None, None, ws, stream), (N, K, M)),
    }
    out = {}
    for name, (run, (m, n, k)) in runs.items():
        for _ in range(5):
            run()
        ms = time_events(run, max(reps, 50), torch)
        fl = 2.0 * m * n * k
        out[name] = {"MxNxK": f"{m}x{n}x{k}", "us": round(ms * 1e3, 2), "TFLOPs": round(fl / (ms * 1e-3) / 1e12, 1),
                     "frac_fp8_peak": round(fl / (ms * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4)}
    return out


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


def stream_ceiling(torch, q, dev, srcs, n_units, dst, sink, reps):
    """The memory-ceiling probe (ql_stream_probe) over the rotated source
    buffers: ms per launch reading 32*n_units bytes and writing 16*n_units
    (dst) or nothing but a 1 MiB sink (read only)."""
    from precision_quantized_gemm_amd import _lib
    stream = torch.cuda.current_stream().cuda_stream
    out = {}
    for name, d, s_ in (("read_2B_write_1B", dst, None), ("read_only", None, sink)):
        i = [0]

        def run():
            _lib.ql_stream_probe(srcs[i[0] % len(srcs)].data_ptr(), n_units, None if d is None else d.data_ptr(),
                              None if s_ is None else s_.data_ptr(), stream)
            i[0] += 1

        for _ in range(len(srcs)):
            run()
        out[name] = time_events(run, reps, torch)
    return out


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
    # Rotated copies of the inputs (the same values at other addresses), so
    # that no input is still in the 256 MB memory-side cache when a timed
    # call reads it: the step alternates between 2 sets of (a, b), 768 MiB;
    # the quantize rates cycle through 3 copies of a (768 MiB) and 5 of b
    # (640 MiB).
    a_sets = [a_cpu.to(dev) for _ in range(3)]
    b_sets = [b_cpu.to(dev) for _ in range(5)]
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

    def gemm():
        q.ql_qgemm(P(x_q), 0, 0, K, P(w_q), 0, 0, K, M, N, K, P(sx), 0, P(sw), 0, None, 0,
                   P(out), _lib.QL_DT_E4M3, N, P(out_scale), P(out_amax), P(ws), stream)

    # The step: one ql_linear_forward call (quantize a and b per tensor, the
    # quantizes sharing each pass's launch, then the GEMM with E4M3 output
    # and out_amax), on input set i % 2.
    def fused_step(i):
        a, b = a_sets[i % 2], b_sets[i % 2]
        q.ql_linear_forward(P(a), _lib.QL_DT_BF16, M, K, P(b), N, None, 0, _lib.QL_FMT_E4M3, None, None,
                            P(out), _lib.QL_DT_E4M3, P(out_scale), P(out_amax), P(x_q), P(sx), P(amax_x),
                            P(w_q), P(sw), P(amax_w), P(ws), stream)

    log("warmup")
    fused_step(0)
    torch.cuda.synchronize()
    out_scale.copy_(out_amax / 448.0)           # amax_prev / 448
    t_w0 = time.perf_counter()
    done = 1
    for i in range(1, max(1, args.warmup)):
        fused_step(i)
    done = max(1, args.warmup)
    torch.cuda.synchronize()
    # Then untimed steps until at least 0.5 s of warm-up have passed, so the
    # clock has settled under this load before the timed region.
    extra = 0
    while time.perf_counter() - t_w0 < 0.5:
        for _ in range(20):
            fused_step(done + extra)
            extra += 1
        torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    ev[0].record()
    for i in range(args.steps):
        fused_step(i)
        ev[i + 1].record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0
    ms_step = ev[0].elapsed_time(ev[-1]) / args.steps
    step_each = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
    pct = lambda xs, f: xs[min(len(xs) - 1, int(f * len(xs)))]

    # Breakdown (after the timed region): the same work as three calls with
    # events between them, for the per-kernel rates and the roofline.
    log("per-call breakdown")

    def step(i, evs=None):
        a, b = a_sets[i % 2], b_sets[i % 2]
        if evs is not None:
            evs[0].record()
        quant(a, M, x_q, sx, amax_x)()
        if evs is not None:
            evs[1].record()
        quant(b, N, w_q, sw, amax_w)()
        if evs is not None:
            evs[2].record()
        gemm()
        if evs is not None:
            evs[3].record()

    for i in range(4):
        step(i)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i, evs in enumerate(events):
        step(i, evs)
    torch.cuda.synchronize()
    ms_step_calls = events[0][0].elapsed_time(events[-1][3]) / args.steps
    ms_gemm = sum(e[2].elapsed_time(e[3]) for e in events) / args.steps
    gemm_each = sorted(e[2].elapsed_time(e[3]) for e in events)
    flops = 2.0 * M * N * K
    value = flops / (ms_step * 1e-3) / 1e12
    gemm_tflops = flops / (ms_gemm * 1e-3) / 1e12

    # Quantize rates on rotated inputs (each call reads a copy that the
    # previous calls have pushed out of the memory-side cache).
    log("quantize on rotated inputs")
    reps_q = max(args.steps, 30)

    def rotating(fn_of, n):
        i = [0]

        def run():
            fn_of(i[0] % n)()
            i[0] += 1
        return run

    qa_rot = rotating(lambda i: quant(a_sets[i], M, x_q, sx, amax_x), len(a_sets))
    qb_rot = rotating(lambda i: quant(b_sets[i], N, w_q, sw, amax_w), len(b_sets))
    for _ in range(6):
        qa_rot(); qb_rot()
    ms_qa = time_events(qa_rot, reps_q, torch)
    ms_qb = time_events(qb_rot, reps_q, torch)

    # Single-pass delayed scaling through an amax history ring (one read of
    # BF16 x, one code byte written: 3 B/elem), on the rotated copies of a.
    ring = torch.zeros(17, dtype=torch.float32, device=dev)
    ring[-1] = 1.0
    su, am = f1(), f1()
    ring_idx = [0]

    def qa_ring_of(i):
        def run():
            q.ql_quantize_ring(P(a_sets[i]), _lib.QL_DT_BF16, M, K, K, _lib.QL_FMT_E4M3, P(ring), 16,
                               ring_idx[0] % 16, 0, P(x_q), K, P(su), P(am), P(ws), stream)
            ring_idx[0] += 1
        return run

    qa_ring = rotating(qa_ring_of, len(a_sets))
    for _ in range(3):
        qa_ring()
    ms_ring = time_events(qa_ring, reps_q, torch)

    # The memory system's ceiling for the same traffic (ql_stream_probe on
    # the same rotated copies of a: 2 B read and 1 B written per element,
    # and read only).
    log("streaming ceiling")
    sink = torch.empty(1 << 20, dtype=u8, device=dev)
    ceil = stream_ceiling(torch, q, dev, a_sets, M * K // 16, x_q, sink, reps_q)

    # Static FP8 inference on the same layer: w arrives quantized (the w_q /
    # sw the step produced), so a call quantizes a and runs the GEMM.
    def static_step_of(i):
        return lambda: q.ql_linear_forward_static(P(a_sets[i]), _lib.QL_DT_BF16, M, K, P(w_q), N, P(sw), None, 0,
                                                  None, _lib.QL_FMT_E4M3, None, P(out), _lib.QL_DT_E4M3,
                                                  P(out_scale), P(out_amax), P(x_q), P(sx), P(amax_x), P(ws),
                                                  stream)

    static_step = rotating(static_step_of, len(a_sets))
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

    log("MLP-up layer products")
    mlp_products = time_mlp_products(torch, q, _lib, synth, dev, args.steps)

    log("per-head batched products")
    per_head = time_per_head(torch, q, _lib, synth, dev, args.steps)

    log("small configurations")
    small = time_configs(torch, q, _lib, synth, dev, args.steps)

    log("INT8 at the benchmark shape")
    int8 = time_int8_large(torch, q, _lib, dev, M, N, K, 10)

    log("shader clock under the GEMM")
    sclk = sclk_under(gemm, torch, 500)

    cpu, cpu_cfg = None, None
    threads = host_threads()
    if not args.no_cpu_baseline:
        log(f"cpu baseline (oracle, {threads} threads)")
        cpu = cpu_baseline(a_cpu, b_cpu, M, N, K, args.cpu_rows, threads)
        log("oracle on the small configurations")
        cpu_cfg = oracle_configs(threads, args.cpu_full)
        gpu_ms = {"tiny_linear": small["tiny_linear"]["ms_eager"], "rowwise_int8": small["rowwise_int8"]["ms_eager"],
                  "mlp_up": small["mlp_up"]["ms_eager"], "mlp_backward": None if bwd is None else bwd["ms_per_call"]}
        for k, v in cpu_cfg.items():
            if gpu_ms.get(k):
                v["gpu_ms"] = gpu_ms[k]
                v["oracle_over_gpu"] = round(v["oracle_s"] * 1e3 / gpu_ms[k], 1)

    qa_bytes3, qa_bytes5 = 3.0 * M * K, 5.0 * M * K
    qb_bytes3, qb_bytes5 = 3.0 * N * K, 5.0 * N * K
    rate = lambda nbytes, ms: nbytes / (ms * 1e-3) / 1e9
    ceil_21 = rate(qa_bytes3, ceil["read_2B_write_1B"])
    ceil_r = rate(2.0 * M * K, ceil["read_only"])
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
                        "(out_scale = amax_prev/448); per step one ql_linear_forward (quantize a and b, the GEMM), "
                        "alternating between 2 copies of the inputs",
            "M": M, "N": N, "K": K, "parallelism": "single GPU",
        },
        "step_ms_p10_p50_p90": [round(pct(step_each, 0.1), 5), round(pct(step_each, 0.5), 5),
                                round(pct(step_each, 0.9), 5)],
        "warmup_extra_steps": extra,
        "roofline": {
            "bound": "mfma",
            "achieved": round(gemm_tflops, 2),
            "peak": PEAK_FP8_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(gemm_tflops / PEAK_FP8_TFLOPS, 4),
            "traffic": gemm_traffic(),
            "kernel": "qgemm_nt_kernel<E4M3,E4M3> (256x256x128 tiles)",
            "ms_per_launch": round(ms_gemm, 5),
            "ms_per_launch_p10_p50_p90": [round(pct(gemm_each, 0.1), 5), round(pct(gemm_each, 0.5), 5),
                                          round(pct(gemm_each, 0.9), 5)],
            "sclk_mhz_under_gemm": sclk,
            "frac_at_measured_sclk": None if not sclk else round(gemm_tflops / (PEAK_FP8_TFLOPS * sclk / 2400.0), 4),
            "per_launch_flops": flops,
        },
        "quantize": {
            "inputs": "rotated: 3 copies of a (768 MiB), 5 of b (640 MiB); none is in the 256 MB memory-side "
                      "cache when its call starts",
            "a_ms": round(ms_qa, 5), "b_ms": round(ms_qb, 5),
            "a_GBps_3B_per_elem": round(rate(qa_bytes3, ms_qa), 1),
            "a_GBps_5B_per_elem": round(rate(qa_bytes5, ms_qa), 1),
            "a_frac_hbm_peak_3B": round(rate(qa_bytes3, ms_qa) / PEAK_HBM_GBPS, 4),
            "a_frac_of_ceiling_3B": round(rate(qa_bytes3, ms_qa) / ceil_21, 4),
            "b_GBps_3B_per_elem": round(rate(qb_bytes3, ms_qb), 1),
            "b_GBps_5B_per_elem": round(rate(qb_bytes5, ms_qb), 1),
            "bytes_per_elem": "per-tensor current scaling reads x twice (amax pass, cast pass) and writes one "
                              "code byte: 5 B; 3 B is the compulsory traffic, against which the *_frac_of_ceiling "
                              "figures compare the rate with the measured 2 B read + 1 B written ceiling",
            "a_ring_ms": round(ms_ring, 5),
            "a_ring_GBps_3B_per_elem": round(rate(qa_bytes3, ms_ring), 1),
            "a_ring_frac_hbm_peak": round(rate(qa_bytes3, ms_ring) / PEAK_HBM_GBPS, 4),
            "a_ring_frac_of_ceiling": round(rate(qa_bytes3, ms_ring) / ceil_21, 4),
            "a_ring_note": "ql_quantize_ring (delayed scaling, 16-entry history): one pass, 3 B/elem",
            "ceiling": {"kernel": "ql_stream_probe (the cast's access pattern, no arithmetic) on the rotated a",
                        "read_2B_write_1B_GBps": round(ceil_21, 1),
                        "read_2B_write_1B_ms": round(ceil["read_2B_write_1B"], 5),
                        "read_only_GBps": round(ceil_r, 1), "read_only_ms": round(ceil["read_only"], 5),
                        "frac_hbm_peak_2to1": round(ceil_21 / PEAK_HBM_GBPS, 4),
                        "frac_hbm_peak_read": round(ceil_r / PEAK_HBM_GBPS, 4)},
            "peak_GBps": PEAK_HBM_GBPS,
        },
        "step_as_three_calls": {"ms_per_step": round(ms_step_calls, 5),
                                "TFLOPs": round(flops / (ms_step_calls * 1e-3) / 1e12, 2),
                                "workload": "the same step as ql_quantize(a), ql_quantize(b), ql_qgemm with events "
                                            "between"},
        "static_inference": {"ms_per_step": round(ms_static, 5),
                             "TFLOPs": round(flops / (ms_static * 1e-3) / 1e12, 2),
                             "workload": "ql_linear_forward_static: quantize a, GEMM with the pre-quantized b"},
        "linear_backward": bwd,
        "mlp_products": mlp_products,
        "per_head": per_head,
        "small_configs": small,
        "int8_large": int8,
        "cpu_baseline": None if cpu is None else {k: (round(v, 6) if isinstance(v, float) else v)
                                                 for k, v in cpu.items()},
        "cpu_baseline_configs": cpu_cfg,
        "wall_s_timed_region": round(t_wall, 4),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
