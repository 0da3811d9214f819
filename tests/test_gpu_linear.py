"""GPU parity of ql_linear_forward (AstrAI ops/fp8.py linear_forward_fp8:
quantize x and w, GEMM with the bias fused) against the oracle's
composition of the same steps."""
import numpy as np
import pytest
import torch

import precision_quantized_gemm_amd as q
from precision_quantized_gemm_amd import synth
from tolerance import check_float, check_fp8_out

pytestmark = pytest.mark.gpu


def _bits(t):
    return synth.bf16_bits(t) if t.dtype == torch.bfloat16 else t.numpy()


def _compare_quant(r, ref):
    assert np.array_equal(r.x_q.cpu().numpy(), ref["x_q"])
    assert np.array_equal(r.w_q.cpu().numpy(), ref["w_q"])
    for k in ("sx", "amax_x", "sw", "amax_w"):
        assert getattr(r, k).cpu().numpy().view(np.uint32)[0] == ref[k].view(np.uint32)[0], k


@pytest.mark.parametrize("name", ["tiny_linear", "mlp_up"])
def test_linear_forward_workloads(orc, name):
    d = synth.workload(name)
    x, w, bias = d["x"], d["w"], d["bias"]
    M, K = x.shape
    N = w.shape[0]
    if name == "tiny_linear":
        ms = ns = None
    else:
        rng = np.random.default_rng(8)
        ms = np.concatenate([np.repeat([5, 1500], N), rng.integers(0, M, 3000)]).astype(np.int64)
        ns = np.concatenate([np.tile(np.arange(N), 2), rng.integers(0, N, 3000)]).astype(np.int64)
    ref = orc.linear_forward(_bits(x), _bits(w), bias.numpy(), orc.E4M3, ms=ms, ns=ns)
    r = q.linear_forward(x.cuda(), w.cuda(), bias.cuda(), "e4m3")
    torch.cuda.synchronize()
    _compare_quant(r, ref)
    got = r.out.cpu().to(torch.float64).numpy()[ref["ms"], ref["ns"]]
    sasb = np.float64(ref["sx"][0]) * np.float64(ref["sw"][0])
    rep = check_float(got, ref["v"], ref["S"], ref["H"], sasb, K, bias=bias.numpy().astype(np.float64)[ref["ns"]],
                      what=name)
    print(name, rep)


def test_linear_forward_delayed_fp8_out_and_int8(orc):
    d = synth.workload("tiny_linear")
    x, w, bias = d["x"], d["w"], d["bias"]
    sx_in = np.array([0.011], np.float32)
    sw_in = np.array([0.0007], np.float32)
    ref = orc.linear_forward(_bits(x), _bits(w), bias.numpy(), orc.E4M3, sx_in=sx_in, sw_in=sw_in)
    os_ = np.float32(np.abs(ref["v"]).max() / 448.0 * 0.7)
    r = q.linear_forward(x.cuda(), w.cuda(), bias.cuda(), "e4m3", sx_in=torch.from_numpy(sx_in).cuda(),
                         sw_in=torch.from_numpy(sw_in).cuda(), out_dtype="e4m3",
                         out_scale=torch.tensor([os_], device="cuda"), out_amax=True)
    torch.cuda.synchronize()
    _compare_quant(r, ref)
    sasb = np.float64(sx_in[0]) * np.float64(sw_in[0])
    differ = check_fp8_out(r.out.cpu().numpy().ravel(), ref["v"], ref["S"], ref["H"], sasb, 128, os_, orc,
                           bias=np.tile(bias.numpy().astype(np.float64), 512), what="delayed fp8 out")
    print("codes differing from enc(exact):", differ)
    # out_amax is max|v| of the FP32 epilogue values: within the float bound of the exact max
    vmax = np.abs(ref["v"]).max()
    assert abs(r.out_amax.item() - vmax) <= 1e-3 * vmax
    # INT8 linear, FP32 in / FP32 out
    xf, wf = x.float(), w.float()
    ref8 = orc.linear_forward(xf.numpy(), wf.numpy(), None, orc.INT8)
    r8 = q.linear_forward(xf.cuda(), wf.cuda(), None, "int8", out_dtype="fp32")
    torch.cuda.synchronize()
    _compare_quant(r8, ref8)
    got = r8.out.cpu().numpy().astype(np.float64).ravel()
    assert np.all(np.abs(got - ref8["v"]) <= 3 * 2.0 ** -24 * np.abs(ref8["v"]))
