"""GPU parity of the pipelined kernel for products with few output tiles
(256 x 128, 128 x 128 or 128 x 64 tiles; csrc/qgemm_pipe.hpp) against the
oracle.

Every shape here gives fewer 256 x 256 tiles than the chip has CUs but at
least one smaller tile per CU, so it takes that kernel: ragged M and N
(partial edge tiles), K tails, both formats and INT8, every layout pair,
per-tensor scales (register epilogue) and per-row scales (LDS epilogue),
E4M3 output with out_amax.  Sampled entries: full rows and columns at the
edges, random entries, and one entry in every output tile.
"""
import numpy as np
import pytest

from precision_quantized_gemm_amd import synth
from tolerance import check_float, check_fp8_out
from test_gpu_qgemm import (finite_codes, storage, run_gpu, out_values, oracle_entries_threaded, per_tile_entries,
                            bias_of)

pytestmark = pytest.mark.gpu


def _entries(M, N, tile_m, tile_n, seed):
    rng = np.random.default_rng(seed)
    rows = np.unique(np.array([0, tile_m - 1, tile_m, M // 2, M - 1]))
    cols = np.unique(np.array([0, tile_n - 1, tile_n, N // 2, N - 1]))
    ms = [np.repeat(rows, N), np.tile(np.arange(M), len(cols)), rng.integers(0, M, 2000)]
    ns = [np.tile(np.arange(N), len(rows)), np.repeat(cols, M), rng.integers(0, N, 2000)]
    tm, tn = np.meshgrid(np.arange(0, M, tile_m), np.arange(0, N, tile_n), indexing="ij")
    ms.append(np.minimum(tm.ravel() + rng.integers(0, tile_m, tm.size), M - 1))
    ns.append(np.minimum(tn.ravel() + rng.integers(0, tile_n, tn.size), N - 1))
    return np.concatenate(ms).astype(np.int64), np.concatenate(ns).astype(np.int64)


def _per_row_entries(orc, a_st, af, al, b_st, bf, bl, K, ms, ns, sa, sb, bias):
    acc, S, iacc, H = orc.qgemm_entries(a_st, af, al, b_st, bf, bl, K, ms, ns)
    v = orc.epilogue(acc, ms, ns, np.asarray(sa, np.float32), 1, np.asarray(sb, np.float32), 1, bias)
    sasb = np.asarray(sa, np.float64)[ms] * np.asarray(sb, np.float64)[ns]
    return acc, S, iacc, H, v, sasb


# (M, N, K, tile): K-major pairs take 128 x 128 tiles, two workgroups per
# CU, with at least two such tiles per CU; else 256 x 128 tiles with one per
# CU; else 128 x 128.
KMAJOR = [(2100, 4000, 1040, (128, 128)), (2048, 4096, 1024, (128, 128)), (2000, 2100, 512, (128, 128)),
          (2064, 4112, 384, (128, 128)), (1920, 4000, 1024, (256, 128)), (1920, 4000, 1040, (256, 128))]


@pytest.mark.parametrize("af,bf", [(0, 0), (1, 0), (0, 1), (2, 2)])
@pytest.mark.parametrize("shape", KMAJOR)
def test_pipe_k_major(orc, af, bf, shape):
    M, N, K, (tm, tn) = shape
    a = finite_codes(orc, 61, af, M, K, af)
    b = finite_codes(orc, 62, bf, N, K, bf)
    ms, ns = _entries(M, N, tm, tn, 63)
    bias = synth.normal(64, 0, N, 0.5)
    sa, sb = [0.004], [0.75]
    if af == 2:
        out = run_gpu(a, 2, 0, b, 2, 0, K, sa, 0, sb, 0, out_dtype="int32")
        _, _, iacc, _ = orc.qgemm_entries(a, 2, 0, b, 2, 0, K, ms, ns)
        assert np.array_equal(out.numpy()[ms, ns].astype(np.int64), iacc)
        return
    acc, S, _, H, v, sasb = oracle_entries_threaded(orc, a, af, 0, b, bf, 0, K, ms, ns, sa, sb)
    v = v + bias.astype(np.float64)[ns]
    out = run_gpu(a, af, 0, b, bf, 0, K, sa, 0, sb, 0, bias=bias, out_dtype="bf16")
    print("pipe k-major", check_float(out_values(out)[ms, ns], v, S, H, sasb, K, bias=bias_of(bias, ns),
                                      what=f"pipe {shape} fmt={af},{bf}"))


# MN-major operands (M, N % 16 == 0): A MN-major, B MN-major, or both.
MN_SHAPES = [(2064, 2048, 1008, 1, 0), (4080, 1040, 2000, 1, 1), (4096, 1024, 2048, 0, 1), (4096, 1024, 2048, 1, 1),
             (384, 19200, 1024, 1, 0), (4128, 1024, 1008, 0, 1)]


@pytest.mark.parametrize("af,bf", [(1, 0), (0, 0), (2, 2)])
@pytest.mark.parametrize("shape", MN_SHAPES)
def test_pipe_mn_major(orc, af, bf, shape):
    M, N, K, al, bl = shape
    a = finite_codes(orc, 71, af * 2 + al, M, K, af)
    b = finite_codes(orc, 72, bf * 2 + bl, N, K, bf)
    a_st, b_st = storage(a, al), storage(b, bl)
    t256 = ((M + 255) // 256) * ((N + 127) // 128)
    tm, tn = (256, 128) if t256 >= 256 else (128, 128)
    ms, ns = _entries(M, N, tm, tn, 73)
    sa, sb = [0.01], [0.02]
    if af == 2:
        out = run_gpu(a_st, 2, al, b_st, 2, bl, K, sa, 0, sb, 0, out_dtype="int32")
        _, _, iacc, _ = orc.qgemm_entries(a_st, 2, al, b_st, 2, bl, K, ms, ns)
        assert np.array_equal(out.numpy()[ms, ns].astype(np.int64), iacc)
        return
    acc, S, _, H, v, sasb = oracle_entries_threaded(orc, a_st, af, al, b_st, bf, bl, K, ms, ns, sa, sb)
    out = run_gpu(a_st, af, al, b_st, bf, bl, K, sa, 0, sb, 0, out_dtype="fp32")
    print("pipe mn", check_float(out_values(out)[ms, ns], v, S, H, sasb, K, what=f"pipe mn {shape} fmt={af},{bf}"))


@pytest.mark.parametrize("al,bl,M", [(0, 0, 1920), (1, 1, 1920), (0, 0, 2100)])
def test_pipe_per_row_and_fp8_out(orc, al, bl, M):
    """Per-row scales take the LDS epilogue with its bounds checks; E4M3
    output with a bias and out_amax takes the register one (256 x 128 tiles,
    and 128 x 128 tiles two workgroups per CU for M = 2100)."""
    N, K = 4000, 768
    a = finite_codes(orc, 81, al, M, K, 0)
    b = finite_codes(orc, 82, bl, N, K, 0)
    a_st, b_st = storage(a, al), storage(b, bl)
    ms, ns = _entries(M, N, 256 if M < 2048 else 128, 128, 83)
    sa = (synth.normal(84, 0, M, 0.1).astype(np.float32) ** 2 + 1e-3).astype(np.float32)
    sb = (synth.normal(84, 1, N, 0.1).astype(np.float32) ** 2 + 1e-3).astype(np.float32)
    bias = synth.normal(85, 0, N, 0.5)
    acc, S, _, H, v, sasb = _per_row_entries(orc, a_st, 0, al, b_st, 0, bl, K, ms, ns, sa, sb, bias)
    out = run_gpu(a_st, 0, al, b_st, 0, bl, K, sa, 1, sb, 1, bias=bias, out_dtype="bf16")
    print("pipe per-row", check_float(out_values(out)[ms, ns], v, S, H, sasb, K, bias=bias_of(bias, ns),
                                      what=f"pipe per-row {al},{bl}"))
    # per-tensor, E4M3 out with bias and out_amax
    acc, S, _, H, v, sasb = oracle_entries_threaded(orc, a_st, 0, al, b_st, 0, bl, K, ms, ns, [0.003], [0.002])
    v = v + bias.astype(np.float64)[ns]
    out32, amax = run_gpu(a_st, 0, al, b_st, 0, bl, K, [0.003], 0, [0.002], 0, bias=bias, out_dtype="fp32",
                          out_amax=True)
    assert amax == np.abs(out32.numpy()).max()
    os_ = np.float32(amax / 448.0)
    out8, amax8 = run_gpu(a_st, 0, al, b_st, 0, bl, K, [0.003], 0, [0.002], 0, bias=bias, out_dtype="e4m3",
                          out_scale=os_, out_amax=True)
    assert amax8 == amax
    differ = check_fp8_out(out8.numpy()[ms, ns], v, S, H, sasb, K, os_, orc, bias=bias_of(bias, ns),
                           what=f"pipe e4m3 {al},{bl}")
    print("pipe e4m3 differing codes:", differ)


# 128 x 64 tiles: single products with fewer 128 x 128 tiles than CUs but
# at least one 128 x 64 tile per CU (the backward's dX shape among them).
T64 = [(2048, 1024, 4096, 0, 1), (2000, 1040, 2048, 1, 1), (1536, 2304, 1024, 0, 1), (2048, 1024, 4096, 1, 0),
       (2048, 1024, 4096, 0, 0), (1900, 1104, 1040, 0, 0)]


@pytest.mark.parametrize("af,bf", [(1, 0), (0, 0), (2, 2)])
@pytest.mark.parametrize("shape", T64)
def test_pipe_128x64(orc, af, bf, shape):
    M, N, K, al, bl = shape
    a = finite_codes(orc, 91, af * 2 + al, M, K, af)
    b = finite_codes(orc, 92, bf * 2 + bl, N, K, bf)
    a_st, b_st = storage(a, al), storage(b, bl)
    ms, ns = _entries(M, N, 128, 64, 93)
    sa, sb = [0.01], [0.02]
    if af == 2:
        out = run_gpu(a_st, 2, al, b_st, 2, bl, K, sa, 0, sb, 0, out_dtype="int32")
        _, _, iacc, _ = orc.qgemm_entries(a_st, 2, al, b_st, 2, bl, K, ms, ns)
        assert np.array_equal(out.numpy()[ms, ns].astype(np.int64), iacc)
        return
    acc, S, _, H, v, sasb = oracle_entries_threaded(orc, a_st, af, al, b_st, bf, bl, K, ms, ns, sa, sb)
    out = run_gpu(a_st, af, al, b_st, bf, bl, K, sa, 0, sb, 0, out_dtype="fp32")
    again = run_gpu(a_st, af, al, b_st, bf, bl, K, sa, 0, sb, 0, out_dtype="fp32")
    assert np.array_equal(out.numpy().view(np.uint32), again.numpy().view(np.uint32)), "result not repeatable"
    print("pipe 128x64", check_float(out_values(out)[ms, ns], v, S, H, sasb, K, what=f"pipe 128x64 {shape} fmt={af},{bf}"))


def test_pipe_128x64_epilogues(orc):
    """128 x 64 tiles with the LDS epilogue (per-row scales, bias, BF16)
    and with E4M3 output and out_amax."""
    M, N, K = 2000, 1040, 2048
    a = finite_codes(orc, 95, 0, M, K, 1)
    b = finite_codes(orc, 96, 1, N, K, 0)
    a_st, b_st = storage(a, 0), storage(b, 1)
    ms, ns = _entries(M, N, 128, 64, 97)
    sa = (synth.normal(98, 0, M, 0.1).astype(np.float32) ** 2 + 1e-3).astype(np.float32)
    sb = (synth.normal(98, 1, N, 0.1).astype(np.float32) ** 2 + 1e-3).astype(np.float32)
    bias = synth.normal(99, 0, N, 0.5)
    acc, S, _, H, v, sasb = _per_row_entries(orc, a_st, 1, 0, b_st, 0, 1, K, ms, ns, sa, sb, bias)
    out = run_gpu(a_st, 1, 0, b_st, 0, 1, K, sa, 1, sb, 1, bias=bias, out_dtype="bf16")
    print("128x64 per-row", check_float(out_values(out)[ms, ns], v, S, H, sasb, K, bias=bias_of(bias, ns),
                                        what="128x64 per-row"))
    acc, S, _, H, v, sasb = oracle_entries_threaded(orc, a_st, 1, 0, b_st, 0, 1, K, ms, ns, [0.003], [0.002])
    v = v + bias.astype(np.float64)[ns]
    out32, amax = run_gpu(a_st, 1, 0, b_st, 0, 1, K, [0.003], 0, [0.002], 0, bias=bias, out_dtype="fp32",
                          out_amax=True)
    assert amax == np.abs(out32.numpy()).max()
    os_ = np.float32(amax / 448.0)
    out8, amax8 = run_gpu(a_st, 1, 0, b_st, 0, 1, K, [0.003], 0, [0.002], 0, bias=bias, out_dtype="e4m3",
                          out_scale=os_, out_amax=True)
    assert amax8 == amax
    print("128x64 e4m3 differing codes:", check_fp8_out(out8.numpy()[ms, ns], v, S, H, sasb, K, os_, orc,
                                                        bias=bias_of(bias, ns), what="128x64 e4m3"))


# More shapes on the pipelined kernel, every output kind of its register
# epilogue.  (M, N, K, tile): two 128 x 128 tiles per CU (two workgroups per
# CU); 544 tiles (the grid does not divide into CUs); twelve steps per
# tile; 272 tiles of 128 x 128 (one workgroup per CU, a second partial
# wave); 384 tiles of 128 x 64.
MORE = [(2048, 4096, 1024, (128, 128)), (2176, 4096, 512, (128, 128)), (1024, 8192, 1536, (128, 128)),
        (2048, 2176, 512, (128, 128)), (2048, 1536, 1024, (128, 64))]


@pytest.mark.parametrize("shape", MORE)
def test_pipe_output_kinds(orc, shape):
    """BF16 with a bias, FP32 with out_amax (exactly max |out|), E4M3 with
    out_amax, mixed formats, and INT8 with raw INT32 output (bit-exact),
    sampled on every tile."""
    M, N, K, (tm, tn) = shape
    ms, ns = _entries(M, N, tm, tn, 101)
    a = finite_codes(orc, 102, 0, M, K, 0)
    b = finite_codes(orc, 103, 0, N, K, 0)
    bias = synth.normal(104, 0, N, 0.5)
    sa, sb = [0.004], [0.75]
    acc, S, _, H, v, sasb = oracle_entries_threaded(orc, a, 0, 0, b, 0, 0, K, ms, ns, sa, sb)
    vb = v + bias.astype(np.float64)[ns]
    out = run_gpu(a, 0, 0, b, 0, 0, K, sa, 0, sb, 0, bias=bias, out_dtype="bf16")
    print("pipe bf16", check_float(out_values(out)[ms, ns], vb, S, H, sasb, K, bias=bias_of(bias, ns),
                                         what=f"pipe {shape} bf16"))
    out32, amax = run_gpu(a, 0, 0, b, 0, 0, K, sa, 0, sb, 0, out_dtype="fp32", out_amax=True)
    check_float(out32.numpy()[ms, ns], v, S, H, sasb, K, what=f"pipe {shape} fp32")
    assert amax == np.abs(out32.numpy()).max()
    os_ = np.float32(amax / 448.0)
    out8, amax8 = run_gpu(a, 0, 0, b, 0, 0, K, sa, 0, sb, 0, out_dtype="e4m3", out_scale=os_, out_amax=True)
    assert amax8 == amax
    check_fp8_out(out8.numpy()[ms, ns], v, S, H, sasb, K, os_, orc, what=f"pipe {shape} e4m3")
    # E5M2 x E4M3
    g = finite_codes(orc, 105, 1, M, K, 1)
    acc, S, _, H, v, sasb = oracle_entries_threaded(orc, g, 1, 0, b, 0, 0, K, ms, ns, sa, sb)
    out = run_gpu(g, 1, 0, b, 0, 0, K, sa, 0, sb, 0, out_dtype="bf16")
    check_float(out_values(out)[ms, ns], v, S, H, sasb, K, what=f"pipe {shape} e5m2 x e4m3")
    # INT8, raw INT32
    ai = finite_codes(orc, 106, 2, M, K, 2)
    bi = finite_codes(orc, 107, 2, N, K, 2)
    outi = run_gpu(ai, 2, 0, bi, 2, 0, K, sa, 0, sb, 0, out_dtype="int32")
    _, _, iacc, _ = orc.qgemm_entries(ai, 2, 0, bi, 2, 0, K, ms, ns)
    assert np.array_equal(outi.numpy()[ms, ns].astype(np.int64), iacc)
