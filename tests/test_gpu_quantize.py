"""GPU parity of ql_quantize against the oracle: bit-exact codes, amax and
scales (AstrAI ops/fp8.py quantize_bf16 / _fp8_quantize_cpu; POPCORNBENCH
"Kimi-K2.6 l2_p13" steps 2-4)."""
import numpy as np
import pytest
import torch

import precision_quantized_gemm_amd as q
from precision_quantized_gemm_amd import _lib, synth

pytestmark = pytest.mark.gpu

FMT = {0: "e4m3", 1: "e5m2", 2: "int8"}
GRAN = {0: "per_tensor", 1: "per_row"}


def _oracle_input(x_cpu):
    return synth.bf16_bits(x_cpu) if x_cpu.dtype == torch.bfloat16 else x_cpu.numpy()


def _gpu(x_cpu, gran, fmt, scale_in=None):
    x = x_cpu.cuda()
    si = None if scale_in is None else torch.from_numpy(np.asarray(scale_in, np.float32).reshape(-1)).cuda()
    xq, s, a = q.quantize(x, GRAN[gran], FMT[fmt], scale_in=si)
    torch.cuda.synchronize()
    return xq.cpu().numpy(), s.cpu().numpy(), a.cpu().numpy()


def _same_codes(got, ref, what):
    if not np.array_equal(got, ref):
        bad = np.argwhere(got != ref)
        raise AssertionError(f"{what}: {len(bad)} codes differ; first {[(tuple(i), hex(got[tuple(i)]), hex(ref[tuple(i)])) for i in bad[:5]]}")


def check(orc, x_cpu, gran, fmt, scale_in=None, what=""):
    got = _gpu(x_cpu, gran, fmt, scale_in)
    ref = orc.quantize(_oracle_input(x_cpu), gran, fmt, scale_in)
    _same_codes(got[0], ref[0], what)
    assert np.array_equal(got[1].view(np.uint32), ref[1].view(np.uint32)), (what, got[1][:4], ref[1][:4])
    assert np.array_equal(got[2].view(np.uint32), ref[2].view(np.uint32)), (what, got[2][:4], ref[2][:4])
    return got


@pytest.mark.parametrize("name,role,gran,fmt", [
    ("tiny_linear", "x", 0, 0), ("tiny_linear", "w", 0, 0),
    ("rowwise_int8", "a", 1, 2), ("rowwise_int8", "b", 1, 2),
    ("mlp_up", "x", 0, 0), ("mlp_up", "w", 0, 0), ("mlp_up", "x", 1, 0),
    ("mlp_backward", "g", 0, 1),
])
def test_workloads(orc, name, role, gran, fmt):
    x = synth.workload(name)[role]
    check(orc, x, gran, fmt, what=f"{name}.{role}")


def _all_bf16():
    bits = np.arange(1 << 16, dtype=np.uint32) << np.uint32(16)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    return torch.from_numpy(f.copy()).to(torch.bfloat16).reshape(1, -1)


@pytest.mark.parametrize("fmt", [0, 1, 2])
@pytest.mark.parametrize("scale", [1.0, 2.0 ** -5, np.float32(3.3) / np.float32(448), np.float32(7) / np.float32(127),
                                   0.0137, 3.0e-30, 2.0 ** -70, 2.0 ** 70, 1.7e25])
def test_every_bf16_value(orc, fmt, scale):
    """All finite BF16 inputs under a given step: the division and the
    round-to-nearest-even encode must match exactly (including steps outside
    the range where the kernel's fast exact division applies)."""
    x = _all_bf16()
    check(orc, x, 0, fmt, np.array([scale], np.float32), what=f"bf16 sweep fmt={fmt} scale={scale}")


@pytest.mark.parametrize("fmt", [0, 1, 2])
def test_fp32_wide_range(orc, fmt):
    rng = np.random.default_rng(100 + fmt)
    n = 1 << 20
    bits = rng.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = np.where(np.isfinite(x), x, np.float32(1.0)).reshape(1024, 1024)
    xt = torch.from_numpy(x.copy())
    for scale in (None, [1.0], [2.0 ** -100], [3.7e-12], [2.0 ** 60]):
        check(orc, xt, 0, fmt, None if scale is None else np.array(scale, np.float32),
              what=f"fp32 wide fmt={fmt} scale={scale}")
    check(orc, xt, 1, fmt, what=f"fp32 wide per-row fmt={fmt}")


SHAPES = [(1, 1), (3, 5), (37, 77), (5, 1000), (64, 16), (130, 33), (2, 4097), (0, 7), (7, 0)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("dt", ["bf16", "fp32"])
def test_ragged_shapes(orc, shape, dt):
    r, c = shape
    x = synth.random_bf16(7, r, r, c, 3.0) if dt == "bf16" else synth.random_fp32(7, r, r, c, 3.0)
    for fmt in (0, 1, 2):
        for gran in (0, 1):
            check(orc, x, gran, fmt, what=f"{shape} {dt} fmt={fmt} gran={gran}")
        check(orc, x, 0, fmt, np.array([0.05], np.float32), what=f"{shape} {dt} fmt={fmt} delayed")
        if r:
            check(orc, x, 1, fmt, np.full(r, 0.03, np.float32), what=f"{shape} {dt} fmt={fmt} delayed per-row")


@pytest.mark.parametrize("ld_extra", [16, 3])
def test_strided_input_and_output(orc, ld_extra):
    """x with ldx > cols (vector rows path when ldx % 16 == 0, scalar
    otherwise) and x_q with ldq > cols through the raw C ABI."""
    rows, cols = 50, 96
    wide = synth.random_bf16(9, ld_extra, rows, cols + ld_extra, 2.0)
    x_cpu = wide[:, :cols]
    ref = orc.quantize(synth.bf16_bits(x_cpu.contiguous()), 0, 0)
    xg = wide.cuda()
    view = xg[:, :cols]
    assert view.stride(0) == cols + ld_extra
    xq_v, s_v, a_v = q.quantize(view, "per_tensor", "e4m3")
    torch.cuda.synchronize()
    _same_codes(xq_v.cpu().numpy(), ref[0], "strided x")
    assert s_v.item() == ref[1][0] and a_v.item() == ref[2][0]
    ldq = cols + 5
    xq = torch.full((rows, ldq), 0xAB, dtype=torch.uint8, device="cuda")
    s = torch.empty(1, device="cuda")
    a = torch.empty(1, device="cuda")
    ws = q.workspace()
    q.ql_quantize(xg.data_ptr(), _lib.QL_DT_BF16, rows, cols, cols + ld_extra, 0, 0, None,
                  xq.data_ptr(), ldq, s.data_ptr(), a.data_ptr(), ws.data_ptr(),
                  torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    out = xq.cpu().numpy()
    _same_codes(out[:, :cols], ref[0], "strided x_q")
    assert (out[:, cols:] == 0xAB).all()
    assert s.item() == ref[1][0] and a.item() == ref[2][0]


def test_workspace_left_reset_across_grid_sizes(orc):
    """The last-workgroup election must leave the workspace zeroed after each
    call, whatever the grid size; amax/scale stay exact over many calls."""
    sizes = [(1, 17), (4096, 1024), (3, 3), (2048, 2048), (1, 1), (333, 4096), (8192, 512)]
    for i in range(3):
        for j, (r, c) in enumerate(sizes):
            x = synth.random_bf16(40 + j, i, r, c, float(1 + j))
            fmt = (i + j) % 3
            delayed = None if (i + j) % 2 else np.array([0.02], np.float32)
            check(orc, x, 0, fmt, delayed, what=f"repeat {i} size {r}x{c}")


def test_empty_tensor_publishes_floor():
    for fmt, floor in ((0, np.float32(1e-12)), (2, np.float32(1e-8))):
        xq, s, a = q.quantize(torch.empty((0, 5), dtype=torch.bfloat16, device="cuda"), "per_tensor", FMT[fmt])
        torch.cuda.synchronize()
        assert a.item() == floor and s.item() == np.float32(floor / np.float32(448 if fmt == 0 else 127))


def test_large_fp8_every_code(orc):
    """The large FP8 workload at full size: every code of both operands."""
    d = synth.workload("large_fp8")
    for role in ("a", "b"):
        check(orc, d[role], 0, 0, what=f"large_fp8.{role}")


@pytest.mark.parametrize("shape,dt,fmt,hist_len", [
    ((1000, 777), "bf16", 0, 4),        # ragged, scalar path
    ((2048, 1024), "bf16", 1, 16),      # flat vector path
    ((513, 2048), "fp32", 2, 3),        # rows path, FP32, INT8
    ((0, 64), "bf16", 0, 2),            # empty: amax is the floor
])
def test_quantize_ring_sequence(orc, shape, dt, fmt, hist_len):
    """Six delayed-scaling steps through one amax history ring: every step's
    codes, the scale they used, amax and the whole ring after the step must
    equal the oracle's bit for bit.  The inputs' spread changes from step to
    step (including a step much smaller than the window's maximum and a
    negative and a positive margin), so the published scale both rises and
    falls as entries leave the window."""
    rows, cols = shape
    ring_ref = np.zeros(hist_len + 1, np.float32)
    ring_ref[-1] = 1.0
    ring = torch.from_numpy(ring_ref.copy()).cuda()
    ws = q.new_workspace(torch.device("cuda"))
    stds = [1.0, 40.0, 0.01, 3.0, 0.5, 1e-3]
    margins = [0, 0, 1, -2, 0, 3]
    for t, (std, margin) in enumerate(zip(stds, margins)):
        idx = t % hist_len
        if dt == "bf16":
            x_cpu = synth.random_bf16(71, t, rows, cols, std)
        else:
            x_cpu = synth.random_fp32(71, t, rows, cols, std)
        xq, su, am = q.quantize_ring(x_cpu.cuda(), FMT[fmt], ring, idx, margin, ws=ws)
        torch.cuda.synchronize()
        codes, su_ref, am_ref = orc.quantize_ring(_oracle_input(x_cpu), fmt, ring_ref, idx, margin)
        _same_codes(xq.cpu().numpy(), codes, f"ring step {t}")
        assert su.item() == su_ref and am.item() == am_ref, (t, su.item(), su_ref, am.item(), am_ref)
        got_ring = ring.cpu().numpy()
        assert np.array_equal(got_ring.view(np.uint32), ring_ref.view(np.uint32)), (t, got_ring, ring_ref)


def test_stream_probe_writes_what_it_reads():
    """The memory-ceiling probe used by the benchmark reads every byte it
    is given: dst[u] = src[2u] XOR src[2u+1] (16-byte words), over a ragged
    number of units and several grid strides."""
    import precision_quantized_gemm_amd._lib as L
    n = 256 * 1024 * 5 + 77
    rng = np.random.default_rng(5)
    src = rng.integers(0, 2 ** 32, size=(n, 8), dtype=np.uint32)
    s = torch.from_numpy(src.view(np.int32)).cuda()
    d = torch.empty((n, 4), dtype=torch.int32, device="cuda")
    sink = torch.empty(1 << 18, dtype=torch.int32, device="cuda")
    L.ql_stream_probe(s.data_ptr(), n, d.data_ptr(), None, torch.cuda.current_stream().cuda_stream)
    L.ql_stream_probe(s.data_ptr(), n, None, sink.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    want = src[:, :4] ^ src[:, 4:]
    assert np.array_equal(d.cpu().numpy().view(np.uint32), want)
