"""CPU oracle for the absmax-scaled quantized linear layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  It shares no
code with the HIP library (``precision_quantized_gemm_amd``) and neither
imports the other; the product path never falls back to it.

The arithmetic lives in ``qlinear_oracle.c`` (plain C, double precision where
the pages leave the precision open).  This module only builds that file with
gcc, loads it with ctypes and marshals numpy arrays.  Each wrapper names the
passage its C function follows; see the C file's header for the sources:

* AstrAI ``astrai/extension/ops/fp8.py`` @ 5e76fbd (module docstring,
  ``_fp8_quantize_cpu``, ``fp8_gemm``/``mm_fp8``/``linear_forward_fp8``
  docstrings),
* POPCORNBENCH "Kimi-K2.6 l2_p13" trace (reference-model steps 2-4 and the
  round-half-to-even discussion),
* scmp_kernels README ("API": per_tensor / per_row, ``a @ b.T``).

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
(codec enumeration, hand-worked fixtures, torch cross-checks, invariants,
brute force).  Nothing is "parity unpinned" except the GPU's FP32
accumulation order inside the matrix cores, which no oracle can fix; it is
bounded by the tolerance instead.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "qlinear_oracle.c"
_LIB = _HERE / "libqlinear_oracle.so"

E4M3, E5M2, INT8 = 0, 1, 2
IN_BF16, IN_FP32 = 0, 1
PER_TENSOR, PER_ROW = 0, 1
K_MAJOR, MN_MAJOR = 0, 1

_lib = None


def build(force: bool = True) -> Path:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not _LIB.exists():
        tmp = _LIB.with_suffix(".so.tmp%d" % os.getpid())
        cmd = ["gcc", "-std=gnu11", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
               "-fno-fast-math", "-Wall", "-Wextra", "-o", str(tmp), str(_SRC), "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def is_stale() -> bool:
    """True when the library is missing or older than its C source."""
    return not _LIB.exists() or _LIB.stat().st_mtime < _SRC.stat().st_mtime


def _load():
    """Load the built library.  Never compiles: a process that may already
    have initialised the GPU must not start a compiler, so a missing or
    stale library is an error here and only ``build()`` (called by the
    package build and at the start of a test session) compiles."""
    global _lib
    if _lib is not None:
        return _lib
    if is_stale():
        raise ImportError(f"{_LIB} is missing or older than {_SRC.name}: run oracle.build() first "
                          "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(str(_LIB))
    i64, i32, dbl, flt, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_float, ctypes.c_void_p
    lib.orc_fp8_encode.argtypes = [dbl, i32]
    lib.orc_fp8_encode.restype = i32
    lib.orc_fp8_decode.argtypes = [i32, i32]
    lib.orc_fp8_decode.restype = dbl
    lib.orc_int8_encode.argtypes = [dbl]
    lib.orc_int8_encode.restype = i32
    lib.orc_div_f32.argtypes = [flt, flt]
    lib.orc_div_f32.restype = flt
    lib.orc_qmax.argtypes = [i32]
    lib.orc_qmax.restype = dbl
    lib.orc_amax_floor.argtypes = [i32]
    lib.orc_amax_floor.restype = flt
    lib.orc_amax_raw.argtypes = [vp, i32, i64, i64, i64, i32, vp]
    lib.orc_amax_raw.restype = None
    lib.orc_quantize.argtypes = [vp, i32, i64, i64, i64, i32, i32, vp, vp, i64, vp, vp]
    lib.orc_quantize.restype = None
    lib.orc_quantize_groups.argtypes = [vp, i32, i64, i64, i64, i64, i32, vp, vp, i64, vp, vp]
    lib.orc_quantize_groups.restype = None
    lib.orc_ring_update.argtypes = [vp, i64, i64, i32, i32, flt]
    lib.orc_ring_update.restype = None
    lib.orc_qgemm_entries.argtypes = [vp, i32, i32, i64, vp, i32, i32, i64, i64, vp, vp, i64, vp, vp, vp, vp, i32, i32]
    lib.orc_qgemm_entries.restype = None
    lib.orc_epilogue.argtypes = [vp, vp, vp, i64, vp, i32, vp, i32, vp, i32, vp]
    lib.orc_epilogue.restype = None
    lib.orc_qbias_values.argtypes = [vp, i64, i32, flt, vp]
    lib.orc_qbias_values.restype = None
    lib.orc_fp8_output.argtypes = [vp, i64, flt, i32, vp]
    lib.orc_fp8_output.restype = None
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


# --------------------------------------------------------------------------
# scalar codecs

def fp8_encode(v: float, fmt: int) -> int:
    """sat(RNE(v)) as an E4M3/E5M2 code (OCP formats, sign of zero kept)."""
    return _load().orc_fp8_encode(float(v), fmt)


def fp8_decode(code: int, fmt: int) -> float:
    """Exact value of an E4M3/E5M2 code."""
    return _load().orc_fp8_decode(int(code), fmt)


def int8_encode(v: float) -> int:
    """clamp(round_half_even(v), -127, 127)."""
    return _load().orc_int8_encode(float(v))


def div_f32(x: float, s: float) -> np.float32:
    """Correctly rounded FP32 quotient x/s."""
    return np.float32(_load().orc_div_f32(float(x), float(s)))


def qmax(fmt: int) -> float:
    return _load().orc_qmax(fmt)


def amax_floor(fmt: int) -> np.float32:
    return np.float32(_load().orc_amax_floor(fmt))


# --------------------------------------------------------------------------
# array entry points

def _input_view(x: np.ndarray):
    """(contiguous array, dtype code) for BF16 bit patterns (uint16) or FP32."""
    if x.dtype == np.uint16:
        return np.ascontiguousarray(x), IN_BF16
    if x.dtype == np.float32:
        return np.ascontiguousarray(x), IN_FP32
    raise TypeError(f"oracle input must be uint16 (BF16 bits) or float32, got {x.dtype}")


def amax_raw(x: np.ndarray, gran: int) -> np.ndarray:
    """max|x| over the tensor ([1]) or each row ([rows]), before any floor."""
    x2, dt = _input_view(x)
    rows, cols = x2.shape
    out = np.zeros(rows if gran == PER_ROW else 1, dtype=np.float64)
    _load().orc_amax_raw(_ptr(x2), dt, rows, cols, cols, gran, _ptr(out))
    return out


def quantize(x: np.ndarray, gran: int, fmt: int, scale_in: np.ndarray | None = None):
    """Return (codes uint8 [rows, cols], scale float32, amax float32).

    ``x`` is a 2-D array of BF16 bit patterns (uint16) or float32.  With
    ``scale_in`` given (delayed scaling) the codes use it; ``scale`` is then
    still fl32(amax/qmax) of this x.
    """
    x2, dt = _input_view(x)
    rows, cols = x2.shape
    n = rows if gran == PER_ROW else 1
    codes = np.zeros((rows, cols), dtype=np.uint8)
    scale = np.zeros(n, dtype=np.float32)
    amax = np.zeros(n, dtype=np.float32)
    sin = None
    if scale_in is not None:
        sin = np.ascontiguousarray(scale_in, dtype=np.float32)
        if sin.size != n:
            raise ValueError("scale_in must hold one value per scale group")
    _load().orc_quantize(_ptr(x2), dt, rows, cols, cols, gran, fmt,
                         _ptr(sin) if sin is not None else None,
                         _ptr(codes), cols, _ptr(scale), _ptr(amax))
    return codes, scale, amax


def quantize_ring(x: np.ndarray, fmt: int, ring: np.ndarray, idx: int, margin: int = 0):
    """One delayed-scaling quantize with an amax history ring.

    ``ring`` is float32 ``[hist_len + 1]`` = ``[hist | scale]`` and is updated
    in place.  Returns ``(codes, scale_used, amax)``: the codes use the
    ring's scale as it was on entry (``scale_used``), ``amax`` (floored) is
    stored at ``hist[idx]`` and the ring's scale becomes the next step's.
    """
    if ring.dtype != np.float32 or ring.ndim != 1 or ring.size < 2:
        raise ValueError("ring must be a 1-D float32 array [hist | scale]")
    hist_len = ring.size - 1
    if not 0 <= idx < hist_len:
        raise ValueError("idx must index the history")
    scale_used = np.float32(ring[hist_len])
    codes, _, amax = quantize(x, PER_TENSOR, fmt, scale_in=np.array([scale_used], np.float32))
    _load().orc_ring_update(_ptr(ring), hist_len, idx, margin, fmt, float(amax[0]))
    return codes, scale_used, np.float32(amax[0])


# Matrix-core alignment used by qgemm_entries' H output: groups of 8
# consecutive products, 13 fraction bits below the group's largest exponent
# sum (measured for the gfx950 FP8 matrix cores; only the acceptance bound
# uses it).
MFMA_GROUP, MFMA_FBITS = 8, 13


def qgemm_entries(a: np.ndarray, a_fmt: int, a_lay: int, b: np.ndarray, b_fmt: int, b_lay: int,
                  K: int, ms: np.ndarray, ns: np.ndarray, group: int = MFMA_GROUP,
                  fbits: int = MFMA_FBITS, with_bound: bool = True):
    """Exact sum_k dec(A[m,k])*dec(B[n,k]) at the listed (m, n) entries.

    ``a``/``b`` are 2-D uint8 code arrays in their storage layout: K-major A
    is [M, K] (ld = a.shape[1]), MN-major A is [K, M].  Returns
    (acc float64, S float64, iacc int64, H float64) where S = sum_k |product|,
    iacc is the integer sum (meaningful for INT8 x INT8) and H bounds the
    truncation of a grouped-alignment accumulator (see the C source; left
    at 0 when ``with_bound`` is false).
    """
    a2 = np.ascontiguousarray(a, dtype=np.uint8)
    b2 = np.ascontiguousarray(b, dtype=np.uint8)
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    if ms.shape != ns.shape:
        raise ValueError("ms and ns must have the same length")
    cnt = ms.size
    acc = np.zeros(cnt, dtype=np.float64)
    sabs = np.zeros(cnt, dtype=np.float64)
    iacc = np.zeros(cnt, dtype=np.int64)
    hb = np.zeros(cnt, dtype=np.float64)
    _load().orc_qgemm_entries(_ptr(a2), a_fmt, a_lay, a2.shape[1], _ptr(b2), b_fmt, b_lay,
                              b2.shape[1], K, _ptr(ms), _ptr(ns), cnt,
                              _ptr(acc), _ptr(sabs), _ptr(iacc), _ptr(hb) if with_bound else None,
                              group, fbits)
    return acc, sabs, iacc, hb


def qgemm_full(a, a_fmt, a_lay, b, b_fmt, b_lay, M, N, K):
    """All M x N entries; returns (acc, S, iacc, H), each [M, N]."""
    mm, nn = np.meshgrid(np.arange(M, dtype=np.int64), np.arange(N, dtype=np.int64), indexing="ij")
    r = qgemm_entries(a, a_fmt, a_lay, b, b_fmt, b_lay, K, mm.ravel(), nn.ravel())
    return tuple(x.reshape(M, N) for x in r)


def epilogue(acc, ms, ns, sa, sa_gran, sb, sb_gran, bias=None):
    """v = acc * sa * sb + bias in double, per entry.  ``bias`` is BF16 bits
    (uint16), float32, or float64 values (a decoded quantized bias)."""
    acc = np.ascontiguousarray(acc, dtype=np.float64)
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    sa = np.ascontiguousarray(sa, dtype=np.float32)
    sb = np.ascontiguousarray(sb, dtype=np.float32)
    out = np.zeros(acc.size, dtype=np.float64)
    bptr, bdt = None, 0
    if bias is not None and np.asarray(bias).dtype == np.float64:
        bias, bdt = np.ascontiguousarray(bias, dtype=np.float64), 2
        bptr = _ptr(bias)
    elif bias is not None:
        bias, bdt = _input_view(np.asarray(bias).reshape(1, -1))
        bptr = _ptr(bias)
    _load().orc_epilogue(_ptr(acc), _ptr(ms), _ptr(ns), acc.size, _ptr(sa), sa_gran,
                         _ptr(sb), sb_gran, bptr, bdt, _ptr(out))
    return out


def fp8_output(v: np.ndarray, out_scale: float, fmt: int = E4M3) -> np.ndarray:
    """sat(RNE(v / out_scale)) as FP8 codes."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    codes = np.zeros(v.size, dtype=np.uint8)
    _load().orc_fp8_output(_ptr(v), v.size, np.float32(out_scale), fmt, _ptr(codes))
    return codes


def fp8_decode_array(codes: np.ndarray, fmt: int) -> np.ndarray:
    """Exact values of an array of FP8 codes (via the 256-entry decode)."""
    table = np.array([fp8_decode(c, fmt) for c in range(256)], dtype=np.float64)
    return table[np.asarray(codes, dtype=np.uint8)]


def linear_forward(x, w, bias, fmt, sx_in=None, sw_in=None, ms=None, ns=None):
    """Quantize x [M,K] and w [N,K] per tensor, then the exact GEMM and the
    epilogue at entries (ms, ns) (all entries when omitted).

    Follows the composition in the ``linear_forward_fp8`` docstring (AstrAI
    ops/fp8.py): quantize x and w to ``fmt``, pre-quantized GEMM with the
    bias fused into the epilogue.  Returns a dict with codes, scales, amax,
    acc, S and v (the reference output values, double).
    """
    xq, sx, ax = quantize(x, PER_TENSOR, fmt, sx_in)
    wq, sw, aw = quantize(w, PER_TENSOR, fmt, sw_in)
    M, K = xq.shape
    N = wq.shape[0]
    if ms is None:
        mm, nn = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
        ms, ns = mm.ravel(), nn.ravel()
    acc, sabs, iacc, hb = qgemm_entries(xq, fmt, K_MAJOR, wq, fmt, K_MAJOR, K, ms, ns)
    sx_used = sx if sx_in is None else np.asarray(sx_in, dtype=np.float32)
    sw_used = sw if sw_in is None else np.asarray(sw_in, dtype=np.float32)
    v = epilogue(acc, ms, ns, sx_used, PER_TENSOR, sw_used, PER_TENSOR, bias)
    return dict(x_q=xq, sx=sx, amax_x=ax, w_q=wq, sw=sw, amax_w=aw,
                acc=acc, S=sabs, iacc=iacc, H=hb, v=v, ms=np.asarray(ms), ns=np.asarray(ns),
                sx_used=sx_used, sw_used=sw_used)


def linear_backward(g, x_q, x_fmt, sx, w_q, w_fmt, sw, g_fmt=E5M2, sg_in=None, dx_entries=None,
                    dw_entries=None):
    """Backward of the quantized linear layer, from the forward's codes.

    Follows the ``linear_backward_fp8`` docstring (AstrAI ops/fp8.py): the
    output gradient g [M, N] is quantized once, per tensor, to ``g_fmt``
    (E5M2 by default), and both products run on codes:
        dX[m, k] = sum_n g[m, n] W[n, k] * sg * sw      ([M, K])
        dW[n, k] = sum_m g[m, n] X[m, k] * sg * sx      ([N, K])
    with x_q [M, K] and w_q [N, K] the forward's codes (the reading of the
    backward workload: E5M2 gradient times the E4M3 forward operands).
    grad_bias[n] = sum_m g[m, n], the column sum of the unquantized gradient
    (math.fsum: exact, then rounded once).  dX and dW are evaluated at the
    listed (m, k) / (n, k) entries (all when None).  Returns a dict with the
    codes, scale and amax of g and, per product, acc / S / H / v.
    """
    import math

    gq, sg, ag = quantize(g, PER_TENSOR, g_fmt, sg_in)
    sg_used = sg if sg_in is None else np.asarray(sg_in, dtype=np.float32)
    M, N = gq.shape
    K = x_q.shape[1]

    def entries(e, rows, cols):
        if e is not None:
            return np.asarray(e[0], np.int64), np.asarray(e[1], np.int64)
        mm, nn = np.meshgrid(np.arange(rows), np.arange(cols), indexing="ij")
        return mm.ravel().astype(np.int64), nn.ravel().astype(np.int64)

    out = dict(g_q=gq, sg=sg, amax_g=ag, sg_used=sg_used)
    # dX: A = g codes [M, N] K-major (contraction n); B[k, n] = W[n, k], i.e.
    # w_q [N, K] read MN-major.
    ms, ks = entries(dx_entries, M, K)
    acc, S, _, H = qgemm_entries(gq, g_fmt, K_MAJOR, w_q, w_fmt, MN_MAJOR, N, ms, ks)
    out["dx"] = dict(ms=ms, ns=ks, acc=acc, S=S, H=H,
                     v=epilogue(acc, ms, ks, sg_used, PER_TENSOR, np.asarray(sw, np.float32), PER_TENSOR))
    # dW: A[n, m] = g[m, n] (g codes read MN-major); B[k, m] = X[m, k]
    # (x_q [M, K] read MN-major); contraction over m.
    ns, ks = entries(dw_entries, N, K)
    acc, S, _, H = qgemm_entries(gq, g_fmt, MN_MAJOR, x_q, x_fmt, MN_MAJOR, M, ns, ks)
    out["dw"] = dict(ms=ns, ns=ks, acc=acc, S=S, H=H,
                     v=epilogue(acc, ns, ks, sg_used, PER_TENSOR, np.asarray(sx, np.float32), PER_TENSOR))
    gv = _input_values(g)
    out["dbias"] = np.array([math.fsum(gv[:, n].tolist()) for n in range(N)], dtype=np.float64)
    return out


def _input_values(x: np.ndarray) -> np.ndarray:
    """BF16 bit patterns (uint16) or float32 as float64 values."""
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def qbias_values(codes: np.ndarray, fmt: int, bias_scale: float) -> np.ndarray:
    """Values of a quantized bias: dec(code) * bias_scale, float64."""
    c = np.ascontiguousarray(codes, dtype=np.uint8).ravel()
    out = np.zeros(c.size, dtype=np.float64)
    _load().orc_qbias_values(_ptr(c), c.size, fmt, float(np.float32(bias_scale)), _ptr(out))
    return out


def linear_forward_static(x, w_q, w_fmt, sw, bias_q, bias_scale, fmt, sx_in=None, ms=None, ns=None):
    """Static FP8 inference ([FP8PY] linear_forward_fp8 docstring): w (and
    optionally the bias) arrive already quantized to ``fmt`` with their steps
    ``sw`` / ``bias_scale``; only x is quantized.  Returns x's codes, step and
    amax and, at entries (ms, ns), acc / S / H / v."""
    xq, sx, ax = quantize(x, PER_TENSOR, fmt, sx_in)
    M, K = xq.shape
    N = w_q.shape[0]
    if ms is None:
        mm, nn = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
        ms, ns = mm.ravel(), nn.ravel()
    acc, S, _, H = qgemm_entries(xq, fmt, K_MAJOR, w_q, w_fmt, K_MAJOR, K, ms, ns)
    sx_used = sx if sx_in is None else np.asarray(sx_in, dtype=np.float32)
    bias = None if bias_q is None else qbias_values(bias_q, fmt, bias_scale)
    v = epilogue(acc, ms, ns, sx_used, PER_TENSOR, np.asarray(sw, np.float32), PER_TENSOR, bias)
    return dict(x_q=xq, sx=sx, amax_x=ax, acc=acc, S=S, H=H, v=v, ms=np.asarray(ms), ns=np.asarray(ns),
                sx_used=sx_used, bias=bias)


def quantize_groups(x: np.ndarray, group_rows: int, fmt: int, scale_in: np.ndarray | None = None):
    """One scale per group of ``group_rows`` consecutive rows ([SCMP] "API"
    group_a / group_b; per_head = N rows of a (BH, N, D) tensor).  Returns
    (codes, scale [ngroups], amax [ngroups])."""
    x2, dt = _input_view(x)
    rows, cols = x2.shape
    if group_rows < 1:
        raise ValueError("group_rows must be >= 1")
    ng = (rows + group_rows - 1) // group_rows
    codes = np.zeros((rows, cols), dtype=np.uint8)
    scale = np.zeros(ng, dtype=np.float32)
    amax = np.zeros(ng, dtype=np.float32)
    sin = None if scale_in is None else np.ascontiguousarray(scale_in, dtype=np.float32)
    _load().orc_quantize_groups(_ptr(x2), dt, rows, cols, cols, group_rows, fmt,
                                _ptr(sin) if sin is not None else None, _ptr(codes), cols, _ptr(scale), _ptr(amax))
    return codes, scale, amax


def qgemm_batched_entries(a, a_fmt, b, b_fmt, zs, ms, ns, sa, group_a, sb, group_b, bias=None):
    """Batched product y[z] = (A[z] @ B[z]^T) with row-group scales, at the
    listed (z, m, n) entries ([SCMP] "API": per_head batches (BH, N, D) and
    N != M; group_a / group_b).  ``a`` is [batch, M, K] codes, ``b``
    [batch, N, K] (both K-major per item).  Scale indices run over the
    flattened rows of all batch items: sa[(z*M + m) // group_a] (group 0 =
    one scale for everything), likewise sb.  Returns (acc, S, H, v) where
    v = acc * sa * sb (+ bias[n]) in double."""
    a = np.ascontiguousarray(a, dtype=np.uint8)
    b = np.ascontiguousarray(b, dtype=np.uint8)
    zs, ms, ns = (np.asarray(t, np.int64) for t in (zs, ms, ns))
    batch, M, K = a.shape
    N = b.shape[1]
    acc = np.zeros(zs.size); S = np.zeros(zs.size); H = np.zeros(zs.size)
    for z in np.unique(zs):
        sel = zs == z
        ac, s_, _, h_ = qgemm_entries(a[z], a_fmt, K_MAJOR, b[z], b_fmt, K_MAJOR, K, ms[sel], ns[sel])
        acc[sel], S[sel], H[sel] = ac, s_, h_
    sa = np.asarray(sa, np.float32).astype(np.float64)
    sb = np.asarray(sb, np.float32).astype(np.float64)
    ia = np.zeros_like(ms) if group_a == 0 else (zs * M + ms) // group_a
    ib = np.zeros_like(ns) if group_b == 0 else (zs * N + ns) // group_b
    v = acc * sa[ia] * sb[ib]
    if bias is not None:
        bv = np.asarray(bias)
        bv = (bv.astype(np.uint32) << 16).view(np.float32) if bv.dtype == np.uint16 else bv.astype(np.float32)
        v = v + bv.astype(np.float64)[ns]
    return acc, S, H, v
