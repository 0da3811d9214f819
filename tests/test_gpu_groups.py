"""GPU parity of the row-group quantize and the batched per-head GEMM
against the oracle ([SCMP] "API": per_head (BH, N, D) products with N != M
for softmax.V; group_a / group_b row-group scales).

Codes, scales and amax of the group quantize are compared bit for bit; the
batched products' float outputs use the bound in tests/tolerance.py and
INT32 accumulators are compared bit for bit.
"""
import numpy as np
import pytest
import torch

import precision_quantized_gemm_amd as q
from precision_quantized_gemm_amd import _lib, synth
from tolerance import check_float, check_fp8_out

pytestmark = pytest.mark.gpu

FMT = {0: "e4m3", 1: "e5m2", 2: "int8"}


def _oracle_input(x_cpu):
    return synth.bf16_bits(x_cpu) if x_cpu.dtype == torch.bfloat16 else x_cpu.numpy()


def _same(got, ref, what):
    if not np.array_equal(got, ref):
        bad = np.argwhere(got != ref)
        raise AssertionError(f"{what}: {len(bad)} differ; first {[(tuple(i), got[tuple(i)], ref[tuple(i)]) for i in bad[:5]]}")


def check_groups(orc, x_cpu, G, fmt, scale_in=None, what=""):
    si = None if scale_in is None else torch.from_numpy(np.asarray(scale_in, np.float32)).cuda()
    xq, s, a = q.quantize_groups(x_cpu.cuda(), G, FMT[fmt], scale_in=si)
    torch.cuda.synchronize()
    x2 = x_cpu.reshape(-1, x_cpu.shape[-1])
    ref = orc.quantize_groups(_oracle_input(x2.contiguous()), G, fmt, scale_in)
    _same(xq.reshape(x2.shape).cpu().numpy(), ref[0], what + " codes")
    _same(s.cpu().numpy().view(np.uint32), ref[1].view(np.uint32), what + " scale")
    _same(a.cpu().numpy().view(np.uint32), ref[2].view(np.uint32), what + " amax")
    return xq, s, a, ref


# ---------------------------------------------------------------------------
# Row-group quantize
@pytest.mark.parametrize("fmt", [0, 1, 2])
@pytest.mark.parametrize("role", ["q", "k", "p", "v"])
def test_per_head_workload_quantize(orc, fmt, role):
    """Each head of the per-head workload (16 heads) gets its own scale."""
    x = synth.workload("per_head")[role]
    check_groups(orc, x, x.shape[1], fmt, what=f"per_head.{role}")


@pytest.mark.parametrize("shape,G", [((1000, 77), 7), ((1000, 77), 1), ((333, 1040), 50), ((64, 16), 64),
                                     ((5, 3), 100), ((4096, 64), 3), ((2, 4097), 1)])
@pytest.mark.parametrize("dt", ["bf16", "fp32"])
def test_groups_ragged(orc, shape, G, dt):
    """Partial last groups, narrow and wide rows, rows with and without a
    16-element vector path, one group larger than the tensor; current and
    delayed (per-group scale_in) scaling, every format."""
    r, c = shape
    x = synth.random_bf16(81, r, r, c, 2.0) if dt == "bf16" else synth.random_fp32(81, r, r, c, 2.0)
    ng = (r + G - 1) // G
    for fmt in (0, 1, 2):
        check_groups(orc, x, G, fmt, what=f"{shape} G={G} {dt} fmt={fmt}")
        check_groups(orc, x, G, fmt, np.linspace(0.01, 0.05, ng).astype(np.float32),
                     what=f"{shape} G={G} {dt} fmt={fmt} delayed")


def test_groups_degenerate(orc):
    """G = 1 equals per-row quantize, G >= rows equals per-tensor; no rows
    launches nothing."""
    x = synth.random_bf16(82, 0, 300, 96, 1.5)
    for fmt in (0, 2):
        _, s1, a1, ref1 = check_groups(orc, x, 1, fmt, what="G=1")
        pr = orc.quantize(_oracle_input(x), 1, fmt)
        _same(ref1[0], pr[0], "G=1 vs per-row")
        _, sT, aT, refT = check_groups(orc, x, 300, fmt, what="G=rows")
        pt = orc.quantize(_oracle_input(x), 0, fmt)
        _same(refT[0], pt[0], "G=rows vs per-tensor")
    xq, s, a = q.quantize_groups(torch.empty((0, 8), dtype=torch.bfloat16, device="cuda"), 4)
    torch.cuda.synchronize()
    assert xq.numel() == 0 and s.numel() == 0


# ---------------------------------------------------------------------------
# Batched per-head GEMM
def _scales_sasb(sa, group_a, sb, group_b, zs, ms, ns, M, N):
    sa = np.asarray(sa, np.float32).astype(np.float64)
    sb = np.asarray(sb, np.float32).astype(np.float64)
    ia = np.zeros_like(ms) if group_a == 0 else (zs * M + ms) // group_a
    ib = np.zeros_like(ns) if group_b == 0 else (zs * N + ns) // group_b
    return sa[ia] * sb[ib]


def _all_zmn(batch, M, N):
    z, m, n = np.meshgrid(np.arange(batch), np.arange(M), np.arange(N), indexing="ij")
    return z.ravel().astype(np.int64), m.ravel().astype(np.int64), n.ravel().astype(np.int64)


def _vals(out):
    return out.to(torch.float64).numpy() if out.dtype == torch.bfloat16 else out.numpy().astype(np.float64)


def _batched_raw(a_st, af, al, lda, sta, b_st, bf, bl, ldb, stb, batch, M, N, K, sa, ga, sb, gb,
                 out_dt="bf16", out_elems=None, ldo=None, sto=None, bias=None, out_scale=None, amax=False):
    """ql_qgemm_batched through the raw C ABI (any layout and stride)."""
    dev = "cuda"
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    A, B = t(a_st), t(b_st)
    tsa, tsb = t(np.asarray(sa, np.float32)), t(np.asarray(sb, np.float32))
    dtc, tdt = {"bf16": (_lib.QL_DT_BF16, torch.bfloat16), "fp32": (_lib.QL_DT_FP32, torch.float32),
                "e4m3": (_lib.QL_DT_E4M3, torch.uint8), "int32": (_lib.QL_DT_INT32, torch.int32)}[out_dt]
    ldo = N if ldo is None else ldo
    sto = M * ldo if sto is None else sto
    out = torch.zeros(batch * sto if out_elems is None else out_elems, dtype=tdt, device=dev)
    tb = None if bias is None else t(bias)
    tos = None if out_scale is None else t(np.asarray([out_scale], np.float32))
    am = torch.zeros(1, dtype=torch.float32, device=dev) if amax else None
    ws = q.workspace() if amax else None
    q.ql_qgemm_batched(A.data_ptr(), af, al, lda, sta, B.data_ptr(), bf, bl, ldb, stb, batch, M, N, K,
                       tsa.data_ptr(), ga, tsb.data_ptr(), gb,
                       None if tb is None else tb.data_ptr(), _lib.QL_DT_FP32 if tb is not None else 0,
                       out.data_ptr(), dtc, ldo, sto, None if tos is None else tos.data_ptr(),
                       None if am is None else am.data_ptr(), None if ws is None else ws.data_ptr(),
                       torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return out.cpu(), (am.item() if amax else None)


def test_per_head_qk(orc):
    """Q.K^T per head on the per-head workload (16 x 196 x 196, D = 64):
    per-head E4M3 scales on both operands, every output entry."""
    d = synth.workload("per_head")
    BH, N, D = d["q"].shape
    qq, sq, _ = orc.quantize_groups(d["q"].reshape(-1, D).numpy(), N, 0)
    kq, sk, _ = orc.quantize_groups(d["k"].reshape(-1, D).numpy(), N, 0)
    a, b = qq.reshape(BH, N, D), kq.reshape(BH, N, D)
    out = q.qgemm_batched(torch.from_numpy(a).cuda(), "e4m3", torch.from_numpy(b).cuda(), "e4m3",
                          torch.from_numpy(sq).cuda(), torch.from_numpy(sk).cuda(), group_a=N, group_b=N)
    torch.cuda.synchronize()
    zs, ms, ns = _all_zmn(BH, N, N)
    acc, S, H, v = orc.qgemm_batched_entries(a, 0, b, 0, zs, ms, ns, sq, N, sk, N)
    got = _vals(out.cpu())[zs, ms, ns]
    print("per-head QK", check_float(got, v, S, H, _scales_sasb(sq, N, sk, N, zs, ms, ns, N, N), D, what="QK"))


@pytest.mark.parametrize("v_fmt", [0, 1])
def test_per_head_softmax_v(orc, v_fmt):
    """P.V per head with N != M: P [16, 196, 160] (per-head E4M3 scales),
    V [16, 160, 64] stored as is, i.e. the MN-major second operand of
    out[z] = P[z] . V[z] (M = 196, N = 64, K = 160), per-head scales on V."""
    d = synth.workload("per_head")
    BH, M, K = d["p"].shape
    N = d["v"].shape[2]
    pq, sp, _ = orc.quantize_groups(d["p"].reshape(-1, K).numpy(), M, 0)
    vq, sv, _ = orc.quantize_groups(d["v"].reshape(-1, N).numpy(), K, v_fmt)
    a = pq.reshape(BH, M, K)
    v_st = vq.reshape(BH, K, N)                               # MN-major storage of B = V^T
    b_log = np.ascontiguousarray(v_st.transpose(0, 2, 1))     # [BH, N, K] for the oracle
    out, _ = _batched_raw(a, 0, _lib.QL_K_MAJOR, K, M * K, v_st, v_fmt, _lib.QL_MN_MAJOR, N, K * N, BH, M, N, K,
                          sp, M, sv, N, out_dt="fp32")
    zs, ms, ns = _all_zmn(BH, M, N)
    acc, S, H, v = orc.qgemm_batched_entries(a, 0, b_log, v_fmt, zs, ms, ns, sp, M, sv, N)
    got = out.numpy().reshape(BH, M, N)[zs, ms, ns].astype(np.float64)
    print("per-head PV", check_float(got, v, S, H, _scales_sasb(sp, M, sv, N, zs, ms, ns, M, N), K, what="PV"))


def _codes(orc, seed, stream, shape, fmt):
    c = synth.random_codes(seed, stream, int(np.prod(shape[:-1])), shape[-1]).reshape(shape)
    if fmt == 2:
        return np.where(c == 0x80, 0, c).astype(np.uint8)
    return np.where(np.isfinite(orc.fp8_decode_array(c, fmt)), c, c & 0x70).astype(np.uint8)


def test_groups_span_items_bias_amax(orc):
    """Row groups that straddle batch items (group_a = 37 over 5 x 100
    rows), one scale for B, an FP32 bias, FP32 output and out_amax over all
    items (equal to max |out|)."""
    batch, M, N, K = 5, 100, 70, 96
    a = _codes(orc, 91, 0, (batch, M, K), 0)
    b = _codes(orc, 91, 1, (batch, N, K), 1)
    ga = 37
    sa = synth.uniform(92, 0, 0, (batch * M + ga - 1) // ga).astype(np.float32) * np.float32(0.01)
    sb = np.array([0.003], np.float32)
    bias = synth.normal(92, 1, N, 0.5)
    out, amax = _batched_raw(a, 0, 0, K, M * K, b, 1, 0, K, N * K, batch, M, N, K, sa, ga, sb, 0,
                             out_dt="fp32", bias=bias, amax=True)
    assert amax == np.abs(out.numpy()).max()
    zs, ms, ns = _all_zmn(batch, M, N)
    acc, S, H, v = orc.qgemm_batched_entries(a, 0, b, 1, zs, ms, ns, sa, ga, sb, 0, bias=bias)
    got = out.numpy().reshape(batch, M, N)[zs, ms, ns].astype(np.float64)
    print("spanning groups", check_float(got, v, S, H, _scales_sasb(sa, ga, sb, 0, zs, ms, ns, M, N), K,
                                         bias=bias[ns].astype(np.float64), what="spanning groups"))


def test_batched_fp8_output(orc):
    """E4M3 output of a batched product: codes within the acceptance set."""
    batch, M, N, K = 3, 130, 200, 256
    a = _codes(orc, 93, 0, (batch, M, K), 0)
    b = _codes(orc, 93, 1, (batch, N, K), 0)
    sa = np.array([0.002, 0.004, 0.001], np.float32)
    sb = np.array([0.003, 0.0015, 0.006], np.float32)
    zs, ms, ns = _all_zmn(batch, M, N)
    acc, S, H, v = orc.qgemm_batched_entries(a, 0, b, 0, zs, ms, ns, sa, M, sb, N)
    os_ = np.float32(np.abs(v).max() / 448.0)
    out, _ = _batched_raw(a, 0, 0, K, M * K, b, 0, 0, K, N * K, batch, M, N, K, sa, M, sb, N,
                          out_dt="e4m3", out_scale=os_)
    got = out.numpy().reshape(batch, M, N)[zs, ms, ns]
    print("batched e4m3 differing:", check_fp8_out(got, v, S, H, _scales_sasb(sa, M, sb, N, zs, ms, ns, M, N), K,
                                                   os_, orc, what="batched e4m3"))


def test_batched_int8_per_head(orc):
    """INT8 per-head batch: INT32 accumulators bit exact for every item."""
    batch, M, N, K = 4, 130, 90, 200
    a = _codes(orc, 94, 0, (batch, M, K), 2)
    b = _codes(orc, 94, 1, (batch, N, K), 2)
    out, _ = _batched_raw(a, 2, 0, K, M * K, b, 2, 0, K, N * K, batch, M, N, K, np.ones(batch, np.float32), M,
                          np.ones(batch, np.float32), N, out_dt="int32")
    zs, ms, ns = _all_zmn(batch, M, N)
    acc, _, _, _ = orc.qgemm_batched_entries(a, 2, b, 2, zs, ms, ns, np.ones(batch), M, np.ones(batch), N)
    assert np.array_equal(out.numpy().reshape(batch, M, N)[zs, ms, ns].astype(np.int64), acc.astype(np.int64))


def test_batched_padded_unaligned_strides(orc):
    """Item strides larger than the item and not multiples of 16 bytes
    (the unaligned staging), an output row pitch above N and an output item
    stride with a gap: the gaps stay untouched."""
    batch, M, N, K = 3, 50, 40, 112
    sta, stb = M * K + 8, N * K + 24
    a_log = _codes(orc, 95, 0, (batch, M, K), 0)
    b_log = _codes(orc, 95, 1, (batch, N, K), 0)
    a_st = np.zeros(batch * sta, np.uint8)
    b_st = np.zeros(batch * stb, np.uint8)
    for z in range(batch):
        a_st[z * sta: z * sta + M * K] = a_log[z].ravel()
        b_st[z * stb: z * stb + N * K] = b_log[z].ravel()
    ldo, sto = N + 3, M * (N + 3) + 5
    sa, sb = np.array([0.01], np.float32), np.array([0.02, 0.03, 0.04], np.float32)
    out, _ = _batched_raw(a_st, 0, 0, K, sta, b_st, 0, 0, K, stb, batch, M, N, K, sa, 0, sb, N,
                          out_dt="fp32", ldo=ldo, sto=sto, out_elems=batch * sto)
    o = out.numpy()
    zs, ms, ns = _all_zmn(batch, M, N)
    got = o[zs * sto + ms * ldo + ns].astype(np.float64)
    acc, S, H, v = orc.qgemm_batched_entries(a_log, 0, b_log, 0, zs, ms, ns, sa, 0, sb, N)
    check_float(got, v, S, H, _scales_sasb(sa, 0, sb, N, zs, ms, ns, M, N), K, what="padded strides")
    written = np.zeros(o.size, bool)
    written[zs * sto + ms * ldo + ns] = True
    assert (o[~written] == 0).all()


def test_groups_on_pipelined_path(orc):
    """batch = 1 with row-group scales on a shape that takes the pipelined
    kernel: the whole tiles use the general epilogue with group indices."""
    M, N, K = 4096 + 37, 4096 + 48, 256
    ga, gb = 100, 300
    a = _codes(orc, 96, 0, (1, M, K), 0)
    b = _codes(orc, 96, 1, (1, N, K), 1)
    sa = synth.uniform(97, 0, 0, (M + ga - 1) // ga).astype(np.float32) * np.float32(0.01)
    sb = synth.uniform(97, 1, 0, (N + gb - 1) // gb).astype(np.float32) * np.float32(0.02)
    out = q.qgemm_batched(torch.from_numpy(a).cuda(), "e4m3", torch.from_numpy(b).cuda(), "e5m2",
                          torch.from_numpy(sa).cuda(), torch.from_numpy(sb).cuda(), group_a=ga, group_b=gb)
    torch.cuda.synchronize()
    rng = np.random.default_rng(98)
    rows = np.array([0, 99, 100, 255, 256, 4095, M - 1])
    cols = np.array([0, 299, 300, 4095, N - 1])
    ms = np.concatenate([np.repeat(rows, N), np.tile(np.arange(M), len(cols)), rng.integers(0, M, 3000)])
    ns = np.concatenate([np.tile(np.arange(N), len(rows)), np.repeat(cols, M), rng.integers(0, N, 3000)])
    ms, ns = ms.astype(np.int64), ns.astype(np.int64)
    zs = np.zeros_like(ms)
    acc, S, H, v = orc.qgemm_batched_entries(a, 0, b, 1, zs, ms, ns, sa, ga, sb, gb)
    got = _vals(out.cpu())[0][ms, ns]
    print("groups on pipelined", check_float(got, v, S, H, _scales_sasb(sa, ga, sb, gb, zs, ms, ns, M, N), K,
                                             what="groups pipelined"))


@pytest.mark.parametrize("al,bl", [(1, 0), (0, 1), (1, 1)])
@pytest.mark.parametrize("pad", [0, 8])
def test_batched_mn_major(orc, al, bl, pad):
    """Batched products with MN-major operands: item strides that keep every
    item 16-byte aligned take the direct-to-LDS kernel, strides padded by 8
    bytes the bounds-checked general kernel; per-item scales on both sides."""
    batch, M, N, K = 3, 48, 80, 96
    a_log = _codes(orc, 101, al, (batch, M, K), 0)
    b_log = _codes(orc, 102, bl, (batch, N, K), 1)

    def pack(log, lay, rows):
        items = [np.ascontiguousarray(log[z] if lay == 0 else log[z].T) for z in range(batch)]
        st = items[0].size + pad
        buf = np.zeros(batch * st, np.uint8)
        for z in range(batch):
            buf[z * st: z * st + items[z].size] = items[z].ravel()
        return buf, st, (K if lay == 0 else rows)

    a_st, sta, lda = pack(a_log, al, M)
    b_st, stb, ldb = pack(b_log, bl, N)
    sa = np.array([0.01, 0.02, 0.005], np.float32)
    sb = np.array([0.03, 0.004, 0.01], np.float32)
    out, _ = _batched_raw(a_st, 0, al, lda, sta, b_st, 1, bl, ldb, stb, batch, M, N, K, sa, M, sb, N, out_dt="fp32")
    zs, ms, ns = _all_zmn(batch, M, N)
    acc, S, H, v = orc.qgemm_batched_entries(a_log, 0, b_log, 1, zs, ms, ns, sa, M, sb, N)
    got = out.numpy().reshape(batch, M, N)[zs, ms, ns].astype(np.float64)
    check_float(got, v, S, H, _scales_sasb(sa, M, sb, N, zs, ms, ns, M, N), K, what=f"batched mn {al},{bl} pad={pad}")
