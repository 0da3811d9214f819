"""ql_linear_forward_noalloc (the allocation-free entry point) against
ql_linear_forward with a caller workspace, through the C ABI.

Two calls of the allocation-free entry point in a row, the second on a
smaller layer, then the same two calls with a workspace: every output must
be identical bit for bit, and both must meet the oracle (codes, steps and
amax bit for bit; float outputs within the float bound, E4M3 outputs in
the acceptance set).
"""
import numpy as np
import pytest
import torch

import precision_quantized_gemm_amd as q
from precision_quantized_gemm_amd import _lib, synth
from tolerance import check_float, check_fp8_out

pytestmark = pytest.mark.gpu


def _layer(name):
    d = synth.workload(name)
    return d["x"], d["w"], d["bias"]


def _run(entry, x, w, bias, out_dtype, out_scale, ws):
    dev = x.device
    M, K = x.shape
    N = w.shape[0]
    odt, tdt = {"bf16": (_lib.QL_DT_BF16, torch.bfloat16), "e4m3": (_lib.QL_DT_E4M3, torch.uint8)}[out_dtype]
    f1 = lambda: torch.full((1,), -1.0, dtype=torch.float32, device=dev)
    r = dict(out=torch.empty((M, N), dtype=tdt, device=dev), x_q=torch.empty((M, K), dtype=torch.uint8, device=dev),
             w_q=torch.empty((N, K), dtype=torch.uint8, device=dev), sx=f1(), amax_x=f1(), sw=f1(), amax_w=f1(),
             out_amax=f1())
    P = lambda t: None if t is None else t.data_ptr()
    args = [P(x), _lib.QL_DT_BF16, M, K, P(w), N, P(bias), _lib.QL_DT_FP32, _lib.QL_FMT_E4M3, None, None,
            P(r["out"]), odt, P(out_scale), P(r["out_amax"]), P(r["x_q"]), P(r["sx"]), P(r["amax_x"]),
            P(r["w_q"]), P(r["sw"]), P(r["amax_w"])]
    stream = torch.cuda.current_stream().cuda_stream
    if entry == "noalloc":
        q.ql_linear_forward_noalloc(*args, stream)
    else:
        q.ql_linear_forward(*args, P(ws), stream)
    return r


def _check_oracle(orc, x, w, bias, r, out_dtype, out_scale, what):
    rng = np.random.default_rng(17)
    M, K = x.shape
    N = w.shape[0]
    ms = np.concatenate([np.repeat([0, M - 1], N), rng.integers(0, M, 3000)]).astype(np.int64)
    ns = np.concatenate([np.tile(np.arange(N), 2), rng.integers(0, N, 3000)]).astype(np.int64)
    ref = orc.linear_forward(synth.bf16_bits(x.cpu()), synth.bf16_bits(w.cpu()), bias.cpu().numpy(), orc.E4M3,
                             ms=ms, ns=ns)
    assert np.array_equal(r["x_q"].cpu().numpy(), ref["x_q"]), what
    assert np.array_equal(r["w_q"].cpu().numpy(), ref["w_q"]), what
    for k in ("sx", "amax_x", "sw", "amax_w"):
        assert r[k].cpu().numpy().view(np.uint32)[0] == ref[k].view(np.uint32)[0], (what, k)
    sasb = np.float64(ref["sx"][0]) * np.float64(ref["sw"][0])
    bias_n = bias.cpu().numpy().astype(np.float64)[ns]
    if out_dtype == "e4m3":
        got = r["out"].cpu().numpy()[ms, ns]
        check_fp8_out(got, ref["v"], ref["S"], ref["H"], sasb, K, float(out_scale.item()), orc, bias=bias_n,
                      what=what)
    else:
        got = r["out"].cpu().to(torch.float64).numpy()[ms, ns]
        check_float(got, ref["v"], ref["S"], ref["H"], sasb, K, bias=bias_n, what=what)


def test_noalloc_matches_workspace_entry(orc):
    dev = torch.device("cuda")
    big = [t.to(dev) for t in _layer("mlp_up")]             # x [2048,1024], W [4096,1024]
    small = [t.to(dev) for t in _layer("tiny_linear")]      # x [512,128], W [128,128]
    os_small = torch.tensor([2.0 ** -6], dtype=torch.float32, device=dev)
    print("[no-alloc] call 1: mlp_up layer, BF16 out", flush=True)
    na1 = _run("noalloc", *big, "bf16", None, None)
    print("[no-alloc] call 2: tiny layer, E4M3 out", flush=True)
    na2 = _run("noalloc", *small, "e4m3", os_small, None)
    torch.cuda.synchronize()
    ws = q.new_workspace(dev)
    w1 = _run("ws", *big, "bf16", None, ws)
    w2 = _run("ws", *small, "e4m3", os_small, ws)
    torch.cuda.synchronize()
    for a, b, what in ((na1, w1, "mlp_up"), (na2, w2, "tiny")):
        for k in a:
            assert torch.equal(a[k].view(torch.uint8), b[k].view(torch.uint8)), (what, k)
    _check_oracle(orc, *big, na1, "bf16", None, "no-alloc mlp_up")
    _check_oracle(orc, *small, na2, "e4m3", os_small, "no-alloc tiny")


def test_noalloc_rejects_bad_arguments():
    """Validation happens before anything is enqueued, as for the
    workspace entry point."""
    f = torch.zeros(4, dtype=torch.float32, device="cuda")
    p = f.data_ptr()
    with pytest.raises(ValueError):          # negative M
        q.ql_linear_forward_noalloc(p, _lib.QL_DT_BF16, -1, 4, p, 4, None, 0, _lib.QL_FMT_E4M3, None, None,
                                    p, _lib.QL_DT_BF16, None, None, p, p, p, p, p, p, 0)
    with pytest.raises(q.QLError):           # a required output missing
        q.ql_linear_forward_noalloc(p, _lib.QL_DT_BF16, 1, 4, p, 1, None, 0, _lib.QL_FMT_E4M3, None, None,
                                    p, _lib.QL_DT_BF16, None, None, p, None, p, p, p, p, 0)
    torch.cuda.synchronize()
    assert torch.count_nonzero(f).item() == 0
