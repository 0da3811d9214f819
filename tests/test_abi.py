"""C-ABI library checks that need no GPU.

* libqlinear.so loads and exports every function include/qlinear.h declares.
* Every argument check fails with its documented status before anything is
  enqueued (no HIP call is reached: with no GPU present, a call that got past
  validation would fail with QL_ERR_HIP instead).
"""
import ctypes
import re
from pathlib import Path

import pytest

import precision_quantized_gemm_amd as q
from precision_quantized_gemm_amd import _lib

ROOT = Path(__file__).resolve().parent.parent
HEADER = ROOT / "include" / "qlinear.h"


def _declared():
    text = re.sub(r"/\*.*?\*/", "", HEADER.read_text(), flags=re.S)
    return sorted(set(re.findall(r"\b(ql_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert _declared() == sorted(["ql_workspace_bytes", "ql_workspace_init", "ql_quantize", "ql_quantize_ring",
                                  "ql_qgemm", "ql_linear_forward", "ql_linear_forward_noalloc", "ql_linear_backward",
                                  "ql_linear_forward_static",
                                  "ql_quantize_groups", "ql_qgemm_batched", "ql_status_string", "ql_last_error"])


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    for name in _declared():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_status_strings_and_workspace_size():
    for s in range(7):
        assert q.ql_status_string(s)
    assert q.ql_status_string(99) == "unknown status"
    assert q.ql_workspace_bytes() >= 16


# A fake but non-NULL device pointer: validation never dereferences it.
P = 1 << 20
Q = (1 << 20) + 4096


def _st(fn, *args):
    lib = _lib.load()
    return getattr(lib, fn)(*args)


def _quant(**kw):
    a = dict(x=P, x_dt=0, rows=4, cols=32, ldx=32, gran=0, fmt=0, scale_in=None, x_q=Q, ldq=32,
             scale_out=P, amax_out=P, ws=P, stream=None)
    a.update(kw)
    return _st("ql_quantize", *a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(x_dt=7), _lib.QL_ERR_VALUE),
    (dict(x_dt=2), _lib.QL_ERR_DTYPE),          # E4M3 is not an input dtype
    (dict(x_dt=3), _lib.QL_ERR_DTYPE),
    (dict(gran=2), _lib.QL_ERR_VALUE),
    (dict(fmt=3), _lib.QL_ERR_VALUE),           # unknown format -> ValueError, as in _fmt_int
    (dict(rows=-1), _lib.QL_ERR_VALUE),
    (dict(cols=-5), _lib.QL_ERR_VALUE),
    (dict(ldx=31), _lib.QL_ERR_SHAPE),
    (dict(ldq=16), _lib.QL_ERR_SHAPE),
    (dict(x=None), _lib.QL_ERR_NULL),
    (dict(x_q=None), _lib.QL_ERR_NULL),
    (dict(scale_out=None), _lib.QL_ERR_NULL),   # current scaling needs it
    (dict(ws=None), _lib.QL_ERR_NULL),          # per-tensor needs the workspace
])
def test_quantize_validation(kw, status):
    assert _quant(**kw) == status
    assert q.ql_last_error()


def _ring(**kw):
    a = dict(x=P, x_dt=0, rows=4, cols=32, ldx=32, fmt=0, ring=P, hist_len=16, idx=3, margin=0, x_q=Q, ldq=32,
             scale_used=P, amax_out=P, ws=P, stream=None)
    a.update(kw)
    return _st("ql_quantize_ring", *a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(ring=None), _lib.QL_ERR_NULL),
    (dict(hist_len=0), _lib.QL_ERR_VALUE),
    (dict(hist_len=(1 << 20) + 1), _lib.QL_ERR_VALUE),
    (dict(idx=16), _lib.QL_ERR_VALUE),
    (dict(idx=-1), _lib.QL_ERR_VALUE),
    (dict(margin=65), _lib.QL_ERR_VALUE),
    (dict(margin=-65), _lib.QL_ERR_VALUE),
    (dict(ws=None), _lib.QL_ERR_NULL),
    (dict(x_dt=1, fmt=4), _lib.QL_ERR_VALUE),
    (dict(x_dt=2), _lib.QL_ERR_DTYPE),
    (dict(ldq=8), _lib.QL_ERR_SHAPE),
    (dict(x_q=None), _lib.QL_ERR_NULL),
])
def test_quantize_ring_validation(kw, status):
    """Every rejected ring call fails before anything is enqueued (no GPU is
    touched: the pointers are never dereferenced)."""
    assert _ring(**kw) == status
    assert q.ql_last_error()


def _gemm(**kw):
    a = dict(a=P, af=0, al=0, lda=64, b=Q, bf=0, bl=0, ldb=64, M=8, N=8, K=64, sa=P, sag=0, sb=P, sbg=0,
             bias=None, bdt=0, out=Q, odt=0, ldo=8, out_scale=None, out_amax=None, ws=None, stream=None)
    a.update(kw)
    return _st("ql_qgemm", *a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(af=5), _lib.QL_ERR_VALUE),
    (dict(af=2, bf=0), _lib.QL_ERR_DTYPE),      # INT8 pairs only with INT8
    (dict(af=1, bf=2), _lib.QL_ERR_DTYPE),
    (dict(al=2), _lib.QL_ERR_VALUE),
    (dict(sag=3), _lib.QL_ERR_VALUE),
    (dict(odt=9), _lib.QL_ERR_VALUE),
    (dict(odt=3), _lib.QL_ERR_DTYPE),           # INT32 output needs INT8 operands
    (dict(M=-1), _lib.QL_ERR_VALUE),
    (dict(af=2, bf=2, K=133145, lda=133145, ldb=133145), _lib.QL_ERR_VALUE),
    (dict(lda=63), _lib.QL_ERR_SHAPE),
    (dict(al=1, lda=7), _lib.QL_ERR_SHAPE),     # MN-major A rows hold M = 8 bytes
    (dict(ldb=10), _lib.QL_ERR_SHAPE),
    (dict(ldo=7), _lib.QL_ERR_SHAPE),
    (dict(a=None), _lib.QL_ERR_NULL),
    (dict(b=None), _lib.QL_ERR_NULL),
    (dict(out=None), _lib.QL_ERR_NULL),
    (dict(sa=None), _lib.QL_ERR_NULL),
    (dict(bias=P, bdt=2), _lib.QL_ERR_DTYPE),
    (dict(odt=2), _lib.QL_ERR_NULL),            # E4M3 output requires out_scale
    (dict(out_amax=P), _lib.QL_ERR_NULL),       # out_amax needs a workspace
])
def test_qgemm_validation(kw, status):
    assert _gemm(**kw) == status


def _linear(**kw):
    a = dict(x=P, xdt=0, M=8, K=64, w=Q, N=8, bias=None, bdt=0, fmt=0, sx_in=None, sw_in=None,
             out=Q, odt=0, out_scale=None, out_amax=None, x_q=P, sx=P, amax_x=P, w_q=Q, sw=P,
             amax_w=P, ws=P, stream=None)
    a.update(kw)
    return _st("ql_linear_forward", *a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(ws=None), _lib.QL_ERR_NULL),
    (dict(sx=None), _lib.QL_ERR_NULL),
    (dict(xdt=2), _lib.QL_ERR_DTYPE),
    (dict(fmt=4), _lib.QL_ERR_VALUE),
    (dict(M=-3), _lib.QL_ERR_VALUE),
    (dict(x_q=None), _lib.QL_ERR_NULL),
    (dict(odt=2), _lib.QL_ERR_NULL),            # E4M3 output without out_scale
    (dict(odt=3), _lib.QL_ERR_DTYPE),           # INT32 output with FP8 operands
])
def test_linear_validation(kw, status):
    assert _linear(**kw) == status


def test_workspace_init_validation():
    assert _st("ql_workspace_init", None, 1024, None) == _lib.QL_ERR_NULL
    assert _st("ql_workspace_init", P, 8, None) == _lib.QL_ERR_VALUE


def test_python_errors_map_to_exceptions():
    with pytest.raises(ValueError):
        q.ql_quantize(P, 0, 4, 32, 31, 0, 0, None, Q, 32, P, P, P)
    with pytest.raises(TypeError):
        q.ql_quantize(P, 2, 4, 32, 32, 0, 0, None, Q, 32, P, P, P)
    with pytest.raises(q.QLError):
        q.ql_quantize(None, 0, 4, 32, 32, 0, 0, None, Q, 32, P, P, P)


def _bwd(**kw):
    a = dict(g=P, M=64, N=32, x_q=Q, x_fmt=0, sx=P, w_q=Q, w_fmt=0, sw=P, K=48, masks=7, g_fmt=1, sg_in=None,
             dx=Q, dw=Q, out_dt=0, dbias=P, g_q=Q, sg=P, amax_g=P, ws=P, stream=None)
    a.update(kw)
    return _st("ql_linear_backward", *a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(masks=0), _lib.QL_ERR_VALUE),
    (dict(masks=8), _lib.QL_ERR_VALUE),
    (dict(out_dt=2), _lib.QL_ERR_DTYPE),          # gradients are BF16 / FP32
    (dict(out_dt=9), _lib.QL_ERR_VALUE),
    (dict(g_fmt=2), _lib.QL_ERR_DTYPE),           # INT8 is not a backward format
    (dict(x_fmt=5), _lib.QL_ERR_VALUE),
    (dict(K=-1), _lib.QL_ERR_VALUE),
    (dict(masks=4, dbias=None), _lib.QL_ERR_NULL),
    (dict(masks=4, ws=None), _lib.QL_ERR_NULL),     # grad_bias's partial sums live in the workspace
    (dict(sg=None), _lib.QL_ERR_NULL),
    (dict(g_q=None), _lib.QL_ERR_NULL),
    (dict(ws=None), _lib.QL_ERR_NULL),
    (dict(masks=1, dx=None), _lib.QL_ERR_NULL),
    (dict(masks=2, dw=None), _lib.QL_ERR_NULL),
    (dict(masks=1, w_q=None), _lib.QL_ERR_NULL),
])
def test_linear_backward_validation(kw, status):
    assert _bwd(**kw) == status
    assert q.ql_last_error()


def _static(**kw):
    a = dict(x=P, x_dt=0, M=64, K=32, w_q=Q, N=48, sw=P, bias=P, bias_dt=1, bias_scale=None, fmt=0, sx_in=None,
             out=Q, out_dt=0, out_scale=None, out_amax=None, x_q=Q, sx=P, amax_x=P, ws=P, stream=None)
    a.update(kw)
    return _st("ql_linear_forward_static", *a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(fmt=2), _lib.QL_ERR_DTYPE),             # static inference is FP8
    (dict(fmt=7), _lib.QL_ERR_VALUE),
    (dict(sw=None), _lib.QL_ERR_NULL),
    (dict(w_q=None), _lib.QL_ERR_NULL),
    (dict(ws=None), _lib.QL_ERR_NULL),
    (dict(sx=None), _lib.QL_ERR_NULL),
    (dict(bias_dt=2), _lib.QL_ERR_DTYPE),         # value bias must be BF16/FP32 without bias_scale
    (dict(out_dt=2), _lib.QL_ERR_NULL),           # E4M3 output needs out_scale
    (dict(x_dt=3), _lib.QL_ERR_DTYPE),
])
def test_linear_forward_static_validation(kw, status):
    assert _static(**kw) == status
    assert q.ql_last_error()


def _groups(**kw):
    a = dict(x=P, x_dt=0, rows=40, cols=32, ldx=32, group_rows=8, fmt=0, scale_in=None, x_q=Q, ldq=32, scale_out=P,
             amax_out=P, stream=None)
    a.update(kw)
    return _st("ql_quantize_groups", *a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(group_rows=0), _lib.QL_ERR_VALUE),
    (dict(group_rows=-3), _lib.QL_ERR_VALUE),
    (dict(fmt=9), _lib.QL_ERR_VALUE),
    (dict(x_dt=2), _lib.QL_ERR_DTYPE),
    (dict(ldx=16), _lib.QL_ERR_SHAPE),
    (dict(x_q=None), _lib.QL_ERR_NULL),
    (dict(scale_out=None), _lib.QL_ERR_NULL),
])
def test_quantize_groups_validation(kw, status):
    assert _groups(**kw) == status
    assert q.ql_last_error()


def _batched(**kw):
    a = dict(a_q=P, a_fmt=0, a_lay=0, lda=64, stride_a=64 * 16, b_q=Q, b_fmt=0, b_lay=0, ldb=64, stride_b=64 * 24,
             batch=4, M=16, N=24, K=64, sa=P, group_a=16, sb=P, group_b=24, bias=None, bias_dt=0, out=Q, out_dt=0,
             ldo=24, stride_out=16 * 24, out_scale=None, out_amax=None, ws=None, stream=None)
    a.update(kw)
    return _st("ql_qgemm_batched", *a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), _lib.QL_ERR_VALUE),
    (dict(batch=65536), _lib.QL_ERR_VALUE),
    (dict(group_a=-1), _lib.QL_ERR_VALUE),
    (dict(stride_b=-5), _lib.QL_ERR_VALUE),
    (dict(a_fmt=2), _lib.QL_ERR_DTYPE),
    (dict(lda=8), _lib.QL_ERR_SHAPE),
    (dict(sa=None), _lib.QL_ERR_NULL),
    (dict(out_dt=2), _lib.QL_ERR_NULL),
    (dict(out_amax=P), _lib.QL_ERR_NULL),      # out_amax needs the workspace
])
def test_qgemm_batched_validation(kw, status):
    assert _batched(**kw) == status
    assert q.ql_last_error()


def test_stream_probe_validates_before_launch():
    """The memory-ceiling probe (include/qlinear_measure.h) rejects bad
    arguments on the host, enqueuing nothing (no GPU needed)."""
    import precision_quantized_gemm_amd._lib as L
    with pytest.raises(ValueError):
        L.ql_stream_probe(16, -1, 32, None)
    with pytest.raises(ValueError):                 # both dst and sink
        L.ql_stream_probe(16, 4, 32, 64)
    with pytest.raises(ValueError):                 # misaligned
        L.ql_stream_probe(8, 4, 32, None)
    with pytest.raises(L.QLError):                  # no source
        L.ql_stream_probe(None, 4, 32, None)
    L.ql_stream_probe(None, 0, None, None)          # nothing to do
