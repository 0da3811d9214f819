"""The last-workgroup election under repetition.

The step of a delayed-scaling quantize is published by the last workgroup
of its single cast pass, and out_amax of a GEMM grid of one wave by the
last workgroup of the GEMM (AstrAI ops/fp8.py @5e76fbd: the commit
message's last-block epilogue; quantize_bf16 and mm_fp8 docstrings).  The
election runs on relaxed device-scope atomics, so these tests repeat it
many times with the maximum planted in a different workgroup's share on
every call, and check each published value exactly against a maximum
computed from the data, and the workspace counters left at zero.
"""
import numpy as np
import pytest
import torch

import precision_quantized_gemm_amd as q
from precision_quantized_gemm_amd import synth

pytestmark = pytest.mark.gpu


def _counters_zero(ws):
    torch.cuda.synchronize()
    head = ws[:1024].cpu().numpy()
    assert not head.any(), np.nonzero(head)[0][:8]


def test_delayed_cast_publishes_every_call():
    """60 delayed-scaling casts of a 4096 x 4096 BF16 tensor (256
    workgroups, one launch each): amax is the planted |value| and the
    published step is fl32(amax / 448), every call."""
    rows, cols = 4096, 4096
    x = synth.random_bf16(91, 0, rows, cols, 1.0).cuda()          # |x| < 8
    ws = q.new_workspace(torch.device("cuda"))
    scale_in = torch.tensor([0.05], dtype=torch.float32, device="cuda")
    rng = np.random.default_rng(12)
    for it in range(60):
        r, c = int(rng.integers(rows)), int(rng.integers(cols))
        v = float(torch.tensor(rng.uniform(16.0, 400.0), dtype=torch.bfloat16)) * (1 if it % 2 else -1)
        old = x[r, c].clone()
        x[r, c] = v
        _, s, a = q.quantize(x, "per_tensor", "e4m3", scale_in=scale_in, ws=ws)
        x[r, c] = old
        want = np.float32(abs(v))
        assert a.item() == want, (it, r, c, a.item(), want)
        assert s.item() == want / np.float32(448.0), (it, s.item())
    _counters_zero(ws)


def test_ring_publishes_every_call():
    """40 ring quantizes (4096 x 2048 FP32, 16-entry history): the stored
    history entry is the planted |value| and the ring's step follows the
    window's maximum."""
    rows, cols = 4096, 2048
    x = synth.random_fp32(92, 0, rows, cols, 1.0).cuda()
    ws = q.new_workspace(torch.device("cuda"))
    hist = 16
    ring = torch.zeros(hist + 1, dtype=torch.float32, device="cuda")
    ring[-1] = 1.0
    ref = np.zeros(hist, np.float32)
    rng = np.random.default_rng(13)
    for it in range(40):
        r, c = int(rng.integers(rows)), int(rng.integers(cols))
        v = np.float32(rng.uniform(10.0, 1000.0))
        old = x[r, c].clone()
        x[r, c] = float(v)
        idx = it % hist
        q.quantize_ring(x, "e4m3", ring, idx, 0, ws=ws)
        x[r, c] = old
        ref[idx] = v
        got = ring.cpu().numpy()
        assert got[idx] == v, (it, got[idx], v)
        assert got[hist] == ref.max() / np.float32(448.0), (it, got[hist], ref.max())
    _counters_zero(ws)


def _e4m3_codes(gen, rows, cols):
    c = torch.randint(0, 256, (rows, cols), generator=gen, device="cuda", dtype=torch.int32).to(torch.uint8)
    return torch.where((c & 0x7F) == 0x7F, c - 1, c)             # no NaN codes


@pytest.mark.parametrize("M,N,K,grid", [
    (4352, 4352, 256, "persistent grid of one workgroup per CU, elected"),
    (2048, 4096, 1024, "pipelined kernel, 512 workgroups, elected"),
    (1000, 1000, 96, "general kernel, small grid, elected"),
    (8192, 8192, 128, "1024 workgroups: per-workgroup maxima and the finalize kernel"),
])
def test_gemm_out_amax_every_call(M, N, K, grid):
    """25 GEMMs with FP32 output and out_amax, the largest product moved to
    another tile on every call: out_amax equals max |out| exactly (both are
    the stored FP32 values)."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(M + N + K)
    a = _e4m3_codes(gen, M, K)
    b = _e4m3_codes(gen, N, K)
    sa = torch.tensor([0.5], dtype=torch.float32, device="cuda")
    sb = torch.tensor([0.25], dtype=torch.float32, device="cuda")
    ws = q.new_workspace(torch.device("cuda"))
    rng = np.random.default_rng(M ^ N ^ K)
    for it in range(25):
        m, n = int(rng.integers(M)), int(rng.integers(N))
        row_a, row_b = a[m].clone(), b[n].clone()
        a[m] = 0x7E                                                  # 448 in every k
        b[n] = 0x7E if it % 2 else 0xFE                              # +-448
        out, amax = q.qgemm(a, "e4m3", b, "e4m3", sa, sb, out_dtype="fp32", out_amax=True, ws=ws)
        a[m], b[n] = row_a, row_b
        want = out.abs().max().item()
        assert amax.item() == want, (grid, it, m, n, amax.item(), want)
        assert abs(out[m, n].item()) == want, (grid, it, out[m, n].item(), want)
    _counters_zero(ws)
