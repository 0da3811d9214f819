"""Torch-tensor front end of the C ABI (argument marshalling only).

PyTorch provides device memory and the stream; each function allocates its
outputs with ``torch.empty`` and calls the matching ``ql_*`` entry point of
libqlinear.so on ``torch.cuda.current_stream()``.  Code tensors are
``torch.uint8`` (view them as ``torch.float8_e4m3fn`` / ``float8_e5m2`` /
``int8`` as needed).  Scales are quantization steps (x_q = x / scale), as in
AstrAI ops/fp8.py @5e76fbd (module docstring); amax is returned fresh.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib
from ._lib import (QL_DT_BF16, QL_DT_E4M3, QL_DT_FP32, QL_DT_INT32, QL_FMT_E4M3, QL_FMT_E5M2,
                   QL_FMT_INT8, QL_K_MAJOR, QL_MN_MAJOR, QL_PER_ROW, QL_PER_TENSOR)

FMTS = {"e4m3": QL_FMT_E4M3, "e5m2": QL_FMT_E5M2, "int8": QL_FMT_INT8}
GRANS = {"per_tensor": QL_PER_TENSOR, "per_row": QL_PER_ROW}
LAYOUTS = {"k_major": QL_K_MAJOR, "mn_major": QL_MN_MAJOR}
_IN_DT = {torch.bfloat16: QL_DT_BF16, torch.float32: QL_DT_FP32}
_OUT_DT = {"bf16": (QL_DT_BF16, torch.bfloat16), "fp32": (QL_DT_FP32, torch.float32),
           "e4m3": (QL_DT_E4M3, torch.uint8), "int32": (QL_DT_INT32, torch.int32)}


def _enum(table, key, what):
    if isinstance(key, int):
        return key
    try:
        return table[key]
    except KeyError:
        raise ValueError(f"unsupported {what} {key!r} (expected one of {sorted(table)})") from None


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


_WORKSPACES: dict = {}


def workspace(device=None) -> torch.Tensor:
    """The default workspace of a device (allocated and zeroed once).

    Calls that share it must be ordered on one stream; give concurrent
    streams their own ``new_workspace()``.
    """
    dev = torch.device(device if device is not None else torch.cuda.current_device())
    if dev.index is None:
        dev = torch.device("cuda", torch.cuda.current_device())
    ws = _WORKSPACES.get(dev.index)
    if ws is None:
        ws = new_workspace(dev)
        _WORKSPACES[dev.index] = ws
    return ws


def new_workspace(device) -> torch.Tensor:
    n = _lib.ql_workspace_bytes()
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    with torch.cuda.device(ws.device):
        _lib.ql_workspace_init(ws.data_ptr(), n, _stream())
    return ws


def _rows_view(x: torch.Tensor):
    if x.dim() != 2:
        raise ValueError(f"expected a 2-D tensor, got shape {tuple(x.shape)}")
    if x.stride(1) != 1 and x.numel() > 0:
        raise ValueError("the last dimension must be contiguous")
    return x.shape[0], x.shape[1], (x.stride(0) if x.shape[0] > 1 else x.shape[1])


def quantize(x: torch.Tensor, granularity="per_tensor", fmt="e4m3", scale_in=None, ws=None):
    """Returns (x_q uint8 [rows, cols], scale float32, amax float32).

    ``scale`` / ``amax`` have one entry per tensor or per row.  With
    ``scale_in`` (delayed scaling) the codes use it and ``scale`` is the step
    of this x (fl32(amax / qmax)).
    """
    if x.dtype not in _IN_DT:
        raise TypeError(f"quantize requires bf16 or fp32 input, got {x.dtype}")
    gran = _enum(GRANS, granularity, "granularity")
    f = _enum(FMTS, fmt, "format")
    rows, cols, ldx = _rows_view(x)
    n = rows if gran == QL_PER_ROW else 1
    x_q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    scale = torch.empty(n, dtype=torch.float32, device=x.device)
    amax = torch.empty(n, dtype=torch.float32, device=x.device)
    if ws is None and gran == QL_PER_TENSOR:
        ws = workspace(x.device)
    _lib.ql_quantize(x.data_ptr(), _IN_DT[x.dtype], rows, cols, ldx, gran, f, _ptr(scale_in),
                     x_q.data_ptr(), cols, scale.data_ptr(), amax.data_ptr(), _ptr(ws), _stream())
    return x_q, scale, amax


def quantize_ring(x: torch.Tensor, fmt, ring: torch.Tensor, idx: int, margin: int = 0, ws=None):
    """Per-tensor delayed scaling with an amax history ring.

    ``ring`` is a float32 device tensor ``[hist_len + 1]`` = ``[hist | scale]``
    updated in place.  Returns ``(x_q, scale_used, amax)``: the codes use the
    ring's scale as it was on entry (``scale_used``, for the GEMM that
    consumes them); ``amax`` is stored at ``hist[idx]`` and the ring's scale
    becomes fl32(max(hist)/qmax) * 2^margin.
    """
    if x.dtype not in _IN_DT:
        raise TypeError(f"quantize_ring requires bf16 or fp32 input, got {x.dtype}")
    if ring.dtype != torch.float32 or ring.dim() != 1 or not ring.is_contiguous():
        raise TypeError("ring must be a contiguous 1-D float32 tensor [hist | scale]")
    f = _enum(FMTS, fmt, "format")
    rows, cols, ldx = _rows_view(x)
    x_q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    scale_used = torch.empty(1, dtype=torch.float32, device=x.device)
    amax = torch.empty(1, dtype=torch.float32, device=x.device)
    if ws is None:
        ws = workspace(x.device)
    _lib.ql_quantize_ring(x.data_ptr(), _IN_DT[x.dtype], rows, cols, ldx, f, ring.data_ptr(), ring.numel() - 1,
                          idx, margin, x_q.data_ptr(), cols, scale_used.data_ptr(), amax.data_ptr(), _ptr(ws),
                          _stream())
    return x_q, scale_used, amax


def quantize_groups(x: torch.Tensor, group_rows: int, fmt="e4m3", scale_in=None):
    """One scale per ``group_rows`` consecutive rows of ``x`` (2-D, or 3-D
    (BH, N, D) flattened to rows: ``group_rows = N`` quantizes per head).
    Returns (x_q with x's shape, scale [ngroups], amax [ngroups])."""
    if x.dtype not in _IN_DT:
        raise TypeError(f"quantize_groups requires bf16 or fp32 input, got {x.dtype}")
    shape = x.shape
    x2 = x.reshape(-1, shape[-1]).contiguous()
    rows, cols = x2.shape
    f = _enum(FMTS, fmt, "format")
    ng = (rows + group_rows - 1) // group_rows if group_rows > 0 else 0
    x_q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    scale = torch.empty(ng, dtype=torch.float32, device=x.device)
    amax = torch.empty(ng, dtype=torch.float32, device=x.device)
    _lib.ql_quantize_groups(x2.data_ptr(), _IN_DT[x.dtype], rows, cols, cols, group_rows, f, _ptr(scale_in),
                            x_q.data_ptr(), cols, scale.data_ptr(), amax.data_ptr(), _stream())
    return x_q.reshape(shape), scale, amax


def qgemm_batched(a_q, a_fmt, b_q, b_fmt, sa, sb, *, group_a=0, group_b=0, bias=None, out_dtype="bf16",
                  out_scale=None, out_amax=False, ws=None):
    """out[z] = (A[z] @ B[z]^T) * sa * sb (+ bias) for K-major codes a_q
    [batch, M, K] and b_q [batch, N, K]; scale of A row m of item z is
    sa[(z*M + m) // group_a] (group_a = M: per head; 0: one scale), likewise
    sb.  Returns out [batch, M, N] or (out, amax)."""
    if a_q.dim() != 3 or b_q.dim() != 3 or a_q.shape[0] != b_q.shape[0] or a_q.shape[2] != b_q.shape[2]:
        raise ValueError("qgemm_batched takes a_q [batch, M, K] and b_q [batch, N, K]")
    a_q, b_q = a_q.contiguous(), b_q.contiguous()
    batch, M, K = a_q.shape
    N = b_q.shape[1]
    odt, tdt = _OUT_DT[out_dtype]
    out = torch.empty((batch, M, N), dtype=tdt, device=a_q.device)
    amax = torch.empty(1, dtype=torch.float32, device=a_q.device) if out_amax else None
    bias_dt = 0
    if bias is not None:
        if bias.dtype not in _IN_DT:
            raise TypeError(f"bias must be bf16 or fp32, got {bias.dtype}")
        bias_dt = _IN_DT[bias.dtype]
    if ws is None and out_amax:
        ws = workspace(a_q.device)
    _lib.ql_qgemm_batched(a_q.data_ptr(), _enum(FMTS, a_fmt, "format"), QL_K_MAJOR, K, M * K,
                          b_q.data_ptr(), _enum(FMTS, b_fmt, "format"), QL_K_MAJOR, K, N * K, batch, M, N, K,
                          _ptr(sa), group_a, _ptr(sb), group_b, _ptr(bias), bias_dt, out.data_ptr(), odt, N, M * N,
                          _ptr(out_scale), _ptr(amax), _ptr(ws), _stream())
    return (out, amax) if out_amax else out


def qgemm(a_q, a_fmt, b_q, b_fmt, sa, sb, *, a_layout="k_major", b_layout="k_major",
          sa_granularity="per_tensor", sb_granularity="per_tensor", bias=None,
          out_dtype="bf16", out_scale=None, out_amax=False, K=None, ws=None):
    """out = (A @ B^T) * sa * sb (+ bias).

    ``a_q`` is the storage of A [M, K]: a [M, K] tensor when K-major or a
    [K, M] tensor when MN-major (likewise ``b_q`` for B [N, K]).  Returns
    ``out`` or ``(out, amax)`` when ``out_amax`` is set.
    """
    af, bf = _enum(FMTS, a_fmt, "format"), _enum(FMTS, b_fmt, "format")
    al, bl = _enum(LAYOUTS, a_layout, "layout"), _enum(LAYOUTS, b_layout, "layout")
    r0, c0, lda = _rows_view(a_q)
    r1, c1, ldb = _rows_view(b_q)
    M, Ka = (r0, c0) if al == QL_K_MAJOR else (c0, r0)
    N, Kb = (r1, c1) if bl == QL_K_MAJOR else (c1, r1)
    if Ka != Kb:
        raise ValueError(f"operand K mismatch: {Ka} vs {Kb}")
    Kd = Ka if K is None else K
    if out_dtype not in _OUT_DT:
        raise ValueError(f"unsupported output dtype {out_dtype!r} (expected one of {sorted(_OUT_DT)})")
    odt, tdt = _OUT_DT[out_dtype]
    out = torch.empty((M, N), dtype=tdt, device=a_q.device)
    amax = torch.empty(1, dtype=torch.float32, device=a_q.device) if out_amax else None
    bias_dt = 0
    if bias is not None:
        if bias.dtype not in _IN_DT:
            raise TypeError(f"bias must be bf16 or fp32, got {bias.dtype}")
        bias_dt = _IN_DT[bias.dtype]
    if ws is None and out_amax:
        ws = workspace(a_q.device)
    _lib.ql_qgemm(a_q.data_ptr(), af, al, lda, b_q.data_ptr(), bf, bl, ldb, M, N, Kd,
                  _ptr(sa), _enum(GRANS, sa_granularity, "granularity"),
                  _ptr(sb), _enum(GRANS, sb_granularity, "granularity"),
                  _ptr(bias), bias_dt, out.data_ptr(), odt, N, _ptr(out_scale), _ptr(amax),
                  _ptr(ws), _stream())
    return (out, amax) if out_amax else out


@dataclass
class LinearOut:
    out: torch.Tensor
    x_q: torch.Tensor
    sx: torch.Tensor
    amax_x: torch.Tensor
    w_q: torch.Tensor
    sw: torch.Tensor
    amax_w: torch.Tensor
    out_amax: Optional[torch.Tensor] = None


def linear_forward(x, w, bias=None, fmt="e4m3", *, sx_in=None, sw_in=None, out_dtype="bf16",
                   out_scale=None, out_amax=False, ws=None) -> LinearOut:
    """Quantize x [M, K] and w [N, K] per tensor, then the scaled GEMM with
    the bias fused (AstrAI ops/fp8.py, linear_forward_fp8)."""
    if x.dtype not in _IN_DT or w.dtype != x.dtype:
        raise TypeError(f"linear_forward requires bf16 or fp32 x and w of the same dtype, got {x.dtype}/{w.dtype}")
    x = x.contiguous()
    w = w.contiguous()
    f = _enum(FMTS, fmt, "format")
    M, K = x.shape
    N, Kw = w.shape
    if Kw != K:
        raise ValueError(f"x is [{M}, {K}] but w is [{N}, {Kw}]")
    if out_dtype not in _OUT_DT:
        raise ValueError(f"unsupported output dtype {out_dtype!r} (expected one of {sorted(_OUT_DT)})")
    odt, tdt = _OUT_DT[out_dtype]
    dev = x.device
    r = LinearOut(
        out=torch.empty((M, N), dtype=tdt, device=dev),
        x_q=torch.empty((M, K), dtype=torch.uint8, device=dev),
        sx=torch.empty(1, dtype=torch.float32, device=dev),
        amax_x=torch.empty(1, dtype=torch.float32, device=dev),
        w_q=torch.empty((N, K), dtype=torch.uint8, device=dev),
        sw=torch.empty(1, dtype=torch.float32, device=dev),
        amax_w=torch.empty(1, dtype=torch.float32, device=dev),
        out_amax=torch.empty(1, dtype=torch.float32, device=dev) if out_amax else None,
    )
    bias_dt = 0
    if bias is not None:
        if bias.dtype not in _IN_DT:
            raise TypeError(f"bias must be bf16 or fp32, got {bias.dtype}")
        bias_dt = _IN_DT[bias.dtype]
    if ws is None:
        ws = workspace(dev)
    _lib.ql_linear_forward(x.data_ptr(), _IN_DT[x.dtype], M, K, w.data_ptr(), N, _ptr(bias), bias_dt, f,
                           _ptr(sx_in), _ptr(sw_in), r.out.data_ptr(), odt, _ptr(out_scale),
                           _ptr(r.out_amax), r.x_q.data_ptr(), r.sx.data_ptr(), r.amax_x.data_ptr(),
                           r.w_q.data_ptr(), r.sw.data_ptr(), r.amax_w.data_ptr(), ws.data_ptr(), _stream())
    return r


def linear_forward_static(x, w_q, sw, bias=None, bias_scale=None, fmt="e4m3", *, sx_in=None, out_dtype="bf16",
                          out_scale=None, out_amax=False, ws=None) -> LinearOut:
    """Static FP8 inference: w arrives quantized (codes ``w_q`` [N, K] of
    ``fmt`` with step ``sw``); ``bias`` is BF16/FP32 values, or codes of
    ``fmt`` when ``bias_scale`` is given.  Only x is quantized.  The result's
    ``w_q``/``sw`` are the inputs and ``amax_w`` is 0 (not measured)."""
    if x.dtype not in _IN_DT:
        raise TypeError(f"linear_forward_static requires bf16 or fp32 x, got {x.dtype}")
    x = x.contiguous()
    f = _enum(FMTS, fmt, "format")
    M, K = x.shape
    N = w_q.shape[0]
    odt, tdt = _OUT_DT[out_dtype]
    dev = x.device
    r = LinearOut(out=torch.empty((M, N), dtype=tdt, device=dev),
                  x_q=torch.empty((M, K), dtype=torch.uint8, device=dev),
                  sx=torch.empty(1, dtype=torch.float32, device=dev),
                  amax_x=torch.empty(1, dtype=torch.float32, device=dev),
                  w_q=w_q, sw=sw, amax_w=torch.zeros(1, dtype=torch.float32, device=dev),
                  out_amax=torch.empty(1, dtype=torch.float32, device=dev) if out_amax else None)
    bias_dt = 0
    if bias is not None and bias_scale is None:
        if bias.dtype not in _IN_DT:
            raise TypeError(f"bias must be bf16 or fp32 values, or codes with bias_scale; got {bias.dtype}")
        bias_dt = _IN_DT[bias.dtype]
    if ws is None:
        ws = workspace(dev)
    _lib.ql_linear_forward_static(x.data_ptr(), _IN_DT[x.dtype], M, K, w_q.data_ptr(), N, sw.data_ptr(),
                                  _ptr(bias), bias_dt, _ptr(bias_scale), f, _ptr(sx_in), r.out.data_ptr(), odt,
                                  _ptr(out_scale), _ptr(r.out_amax), r.x_q.data_ptr(), r.sx.data_ptr(),
                                  r.amax_x.data_ptr(), ws.data_ptr(), _stream())
    return r


@dataclass
class LinearGrads:
    dx: Optional[torch.Tensor]
    dw: Optional[torch.Tensor]
    dbias: Optional[torch.Tensor]
    g_q: Optional[torch.Tensor]
    sg: Optional[torch.Tensor]
    amax_g: Optional[torch.Tensor]


def linear_backward(g, x_q, sx, w_q, sw, *, x_fmt="e4m3", w_fmt="e4m3", g_fmt="e5m2",
                    masks=(True, True, True), sg_in=None, out_dtype="bf16", ws=None) -> LinearGrads:
    """Backward of the quantized linear layer from the forward's codes.

    ``g`` is the BF16 output gradient [M, N]; ``x_q`` [M, K] / ``w_q`` [N, K]
    and their steps ``sx`` / ``sw`` come from the forward.  ``masks`` picks
    (dX, dW, grad_bias).  g is quantized once to ``g_fmt`` for both products.
    """
    if g.dtype != torch.bfloat16:
        raise TypeError(f"linear_backward requires a bf16 gradient, got {g.dtype}")
    M, N = g.shape
    K = x_q.shape[1]
    dev = g.device
    want_dx, want_dw, want_db = (bool(m) for m in masks)
    bits = (_lib.QL_BWD_DX if want_dx else 0) | (_lib.QL_BWD_DW if want_dw else 0) | \
        (_lib.QL_BWD_DBIAS if want_db else 0)
    if out_dtype not in ("bf16", "fp32"):
        raise ValueError("linear_backward writes bf16 or fp32 gradients")
    odt, tdt = _OUT_DT[out_dtype]
    gemms = want_dx or want_dw
    dx = torch.empty((M, K), dtype=tdt, device=dev) if want_dx else None
    dw = torch.empty((N, K), dtype=tdt, device=dev) if want_dw else None
    dbias = torch.empty(N, dtype=torch.float32, device=dev) if want_db else None
    g_q = torch.empty((M, N), dtype=torch.uint8, device=dev) if gemms else None
    sg = torch.empty(1, dtype=torch.float32, device=dev) if gemms else None
    amax_g = torch.empty(1, dtype=torch.float32, device=dev) if gemms else None
    if ws is None:
        ws = workspace(dev)
    g = g.contiguous()
    _lib.ql_linear_backward(g.data_ptr(), M, N, x_q.data_ptr(), _enum(FMTS, x_fmt, "format"), sx.data_ptr(),
                            w_q.data_ptr(), _enum(FMTS, w_fmt, "format"), sw.data_ptr(), K, bits,
                            _enum(FMTS, g_fmt, "format"), _ptr(sg_in), _ptr(dx), _ptr(dw), odt, _ptr(dbias),
                            _ptr(g_q), _ptr(sg), _ptr(amax_g), _ptr(ws), _stream())
    return LinearGrads(dx, dw, dbias, g_q, sg, amax_g)
