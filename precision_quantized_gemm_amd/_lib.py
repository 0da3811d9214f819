"""ctypes binding of libqlinear.so (include/qlinear.h).

The ``ql_*`` functions take the C-ABI's arguments one to one (device
pointers as Python ints, sizes, enum values) and only marshal them; every
step of the quantized linear layer runs in the HIP kernels behind them.
A non-OK status raises: ValueError for QL_ERR_VALUE / QL_ERR_SHAPE,
TypeError for QL_ERR_DTYPE, RuntimeError otherwise.

The library must have been built (``precision_quantized_gemm_amd.build``);
there is no fallback of any kind when it is missing.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

LIB_PATH = Path(__file__).resolve().parent / "libqlinear.so"

# enums (include/qlinear.h)
QL_OK, QL_ERR_VALUE, QL_ERR_DTYPE, QL_ERR_SHAPE, QL_ERR_NULL, QL_ERR_UNSUPPORTED, QL_ERR_HIP = range(7)
QL_FMT_E4M3, QL_FMT_E5M2, QL_FMT_INT8 = 0, 1, 2
QL_DT_BF16, QL_DT_FP32, QL_DT_E4M3, QL_DT_INT32 = 0, 1, 2, 3
QL_PER_TENSOR, QL_PER_ROW = 0, 1
QL_K_MAJOR, QL_MN_MAJOR = 0, 1

_lib = None


class QLError(RuntimeError):
    """A HIP-side failure (QL_ERR_NULL / UNSUPPORTED / HIP)."""

    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def load():
    """Load libqlinear.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not LIB_PATH.exists():
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m precision_quantized_gemm_amd.build` "
            "(there is no CPU fallback)")
    lib = ctypes.CDLL(str(LIB_PATH))
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    lib.ql_workspace_bytes.argtypes = []
    lib.ql_workspace_bytes.restype = sz
    lib.ql_workspace_init.argtypes = [vp, sz, vp]
    lib.ql_workspace_init.restype = i32
    lib.ql_quantize.argtypes = [vp, i32, i64, i64, i64, i32, i32, vp, vp, i64, vp, vp, vp, vp]
    lib.ql_quantize.restype = i32
    lib.ql_quantize_ring.argtypes = [vp, i32, i64, i64, i64, i32, vp, i64, i64, i32, vp, i64, vp, vp, vp, vp]
    lib.ql_quantize_ring.restype = i32
    lib.ql_qgemm.argtypes = [vp, i32, i32, i64, vp, i32, i32, i64, i64, i64, i64,
                             vp, i32, vp, i32, vp, i32, vp, i32, i64, vp, vp, vp, vp]
    lib.ql_qgemm.restype = i32
    lib.ql_linear_forward.argtypes = [vp, i32, i64, i64, vp, i64, vp, i32, i32, vp, vp,
                                      vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.ql_linear_forward.restype = i32
    lib.ql_linear_forward_noalloc.argtypes = [vp, i32, i64, i64, vp, i64, vp, i32, i32, vp, vp,
                                              vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.ql_linear_forward_noalloc.restype = i32
    lib.ql_quantize_groups.argtypes = [vp, i32, i64, i64, i64, i64, i32, vp, vp, i64, vp, vp, vp]
    lib.ql_quantize_groups.restype = i32
    lib.ql_qgemm_batched.argtypes = [vp, i32, i32, i64, i64, vp, i32, i32, i64, i64, i64, i64, i64, i64,
                                     vp, i64, vp, i64, vp, i32, vp, i32, i64, i64, vp, vp, vp, vp]
    lib.ql_qgemm_batched.restype = i32
    lib.ql_linear_forward_static.argtypes = [vp, i32, i64, i64, vp, i64, vp, vp, i32, vp, i32, vp,
                                             vp, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.ql_linear_forward_static.restype = i32
    lib.ql_linear_backward.argtypes = [vp, i64, i64, vp, i32, vp, vp, i32, vp, i64, ctypes.c_uint, i32, vp,
                                       vp, vp, i32, vp, vp, vp, vp, vp, vp]
    lib.ql_linear_backward.restype = i32
    lib.ql_stream_probe.argtypes = [vp, i64, vp, vp, vp]
    lib.ql_stream_probe.restype = i32
    lib.ql_status_string.argtypes = [i32]
    lib.ql_status_string.restype = ctypes.c_char_p
    lib.ql_last_error.argtypes = []
    lib.ql_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int, what: str) -> None:
    if status == QL_OK:
        return
    lib = load()
    msg = f"{what}: {lib.ql_status_string(status).decode()}: {lib.ql_last_error().decode()}"
    if status in (QL_ERR_VALUE, QL_ERR_SHAPE):
        raise ValueError(msg)
    if status == QL_ERR_DTYPE:
        raise TypeError(msg)
    raise QLError(status, msg)


def ql_workspace_bytes() -> int:
    return int(load().ql_workspace_bytes())


def ql_workspace_init(ws: int, nbytes: int, stream: int = 0) -> None:
    _check(load().ql_workspace_init(ws, nbytes, stream), "ql_workspace_init")


def ql_quantize(x, x_dt, rows, cols, ldx, gran, fmt, scale_in, x_q, ldq, scale_out, amax_out,
                ws, stream=0) -> None:
    _check(load().ql_quantize(x, x_dt, rows, cols, ldx, gran, fmt, scale_in, x_q, ldq,
                              scale_out, amax_out, ws, stream), "ql_quantize")


def ql_quantize_ring(x, x_dt, rows, cols, ldx, fmt, ring, hist_len, idx, margin, x_q, ldq, scale_used,
                     amax_out, ws, stream=0) -> None:
    _check(load().ql_quantize_ring(x, x_dt, rows, cols, ldx, fmt, ring, hist_len, idx, margin, x_q, ldq,
                                   scale_used, amax_out, ws, stream), "ql_quantize_ring")


def ql_qgemm(a_q, a_fmt, a_lay, lda, b_q, b_fmt, b_lay, ldb, M, N, K, sa, sa_gran, sb, sb_gran,
             bias, bias_dt, out, out_dt, ldo, out_scale, out_amax, ws, stream=0) -> None:
    _check(load().ql_qgemm(a_q, a_fmt, a_lay, lda, b_q, b_fmt, b_lay, ldb, M, N, K, sa, sa_gran,
                           sb, sb_gran, bias, bias_dt, out, out_dt, ldo, out_scale, out_amax,
                           ws, stream), "ql_qgemm")


def ql_linear_forward(x, x_dt, M, K, w, N, bias, bias_dt, fmt, sx_in, sw_in, out, out_dt,
                      out_scale, out_amax, x_q, sx, amax_x, w_q, sw, amax_w, ws, stream=0) -> None:
    _check(load().ql_linear_forward(x, x_dt, M, K, w, N, bias, bias_dt, fmt, sx_in, sw_in, out,
                                    out_dt, out_scale, out_amax, x_q, sx, amax_x, w_q, sw, amax_w,
                                    ws, stream), "ql_linear_forward")


def ql_linear_forward_noalloc(x, x_dt, M, K, w, N, bias, bias_dt, fmt, sx_in, sw_in, out, out_dt,
                              out_scale, out_amax, x_q, sx, amax_x, w_q, sw, amax_w, stream=0) -> None:
    _check(load().ql_linear_forward_noalloc(x, x_dt, M, K, w, N, bias, bias_dt, fmt, sx_in, sw_in, out,
                                            out_dt, out_scale, out_amax, x_q, sx, amax_x, w_q, sw, amax_w,
                                            stream), "ql_linear_forward_noalloc")


def ql_quantize_groups(x, x_dt, rows, cols, ldx, group_rows, fmt, scale_in, x_q, ldq, scale_out, amax_out,
                       stream=0) -> None:
    _check(load().ql_quantize_groups(x, x_dt, rows, cols, ldx, group_rows, fmt, scale_in, x_q, ldq, scale_out,
                                     amax_out, stream), "ql_quantize_groups")


def ql_qgemm_batched(a_q, a_fmt, a_lay, lda, stride_a, b_q, b_fmt, b_lay, ldb, stride_b, batch, M, N, K,
                     sa, group_a, sb, group_b, bias, bias_dt, out, out_dt, ldo, stride_out, out_scale, out_amax,
                     ws, stream=0) -> None:
    _check(load().ql_qgemm_batched(a_q, a_fmt, a_lay, lda, stride_a, b_q, b_fmt, b_lay, ldb, stride_b, batch, M,
                                   N, K, sa, group_a, sb, group_b, bias, bias_dt, out, out_dt, ldo, stride_out,
                                   out_scale, out_amax, ws, stream), "ql_qgemm_batched")


def ql_linear_forward_static(x, x_dt, M, K, w_q, N, sw, bias, bias_dt, bias_scale, fmt, sx_in, out, out_dt,
                             out_scale, out_amax, x_q, sx, amax_x, ws, stream=0) -> None:
    _check(load().ql_linear_forward_static(x, x_dt, M, K, w_q, N, sw, bias, bias_dt, bias_scale, fmt, sx_in, out,
                                           out_dt, out_scale, out_amax, x_q, sx, amax_x, ws, stream),
           "ql_linear_forward_static")


QL_BWD_DX, QL_BWD_DW, QL_BWD_DBIAS = 1, 2, 4


def ql_linear_backward(g, M, N, x_q, x_fmt, sx, w_q, w_fmt, sw, K, masks, g_fmt, sg_in, dx, dw, out_dt, dbias,
                       g_q, sg, amax_g, ws, stream=0) -> None:
    _check(load().ql_linear_backward(g, M, N, x_q, x_fmt, sx, w_q, w_fmt, sw, K, masks, g_fmt, sg_in, dx, dw,
                                     out_dt, dbias, g_q, sg, amax_g, ws, stream), "ql_linear_backward")


def ql_stream_probe(src, n_units, dst, sink, stream=0) -> None:
    """The memory-ceiling probe of include/qlinear_measure.h (a measurement
    aid outside the method)."""
    _check(load().ql_stream_probe(src, n_units, dst, sink, stream), "ql_stream_probe")


def ql_status_string(status: int) -> str:
    return load().ql_status_string(status).decode()


def ql_last_error() -> str:
    return load().ql_last_error().decode()
