/*
 * qlinear.h -- C ABI of the MI355X (gfx950) absmax-scaled quantized linear
 * layer: a fused quantize pass and a scaled FP8/INT8 matrix-core GEMM.
 *
 * Sources (web pages, cited by title and section):
 *   [FP8PY]  AstrAI, astrai/extension/ops/fp8.py at commit 5e76fbd: the module
 *            docstring (primitives, scale semantics), quantize_bf16, mm_fp8 /
 *            fp8_gemm, linear_forward_fp8, and the commit message (last-block
 *            scale epilogue, no zero-fill dispatch, grouped rasterization).
 *   [TRACE]  POPCORNBENCH page "Kimi-K2.6 l2_p13": the reference model's
 *            symmetric INT8 steps (amax clamp, scale = amax/127, clamp to
 *            +-127, round half to even) and the device-resident scale.
 *   [SCMP]   CrucibleComputingGroup/scmp_kernels README, "API": per_tensor /
 *            per_row granularity, a @ b.T orientation.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor pointer is a DEVICE pointer on the current HIP device;
 *   sizes and leading dimensions are in elements.  Matrices are row-major
 *   with the given leading dimension (distance between consecutive rows).
 * - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *   All device work is enqueued on it; no call synchronizes the host and no
 *   call allocates device memory.
 * - The caller owns every buffer, including the workspace.  The library
 *   keeps no global mutable state besides a thread-local error string and,
 *   for ql_linear_forward_noalloc only, that call's device scratch array
 *   and the cache of its per-device address.
 * - Scales are quantization STEPS: codes are x / scale ([FP8PY] module
 *   docstring).  The library forms any reciprocal itself.  amax values are
 *   outputs only, never accumulated into, so callers never clear them.
 * - Errors: arguments are validated on the host before anything is
 *   enqueued.  On any error nothing is enqueued, outputs are untouched and
 *   ql_last_error() describes the problem.  QL_ERR_VALUE mirrors a Python
 *   ValueError (bad enum, bad size), QL_ERR_DTYPE a TypeError (a dtype or
 *   format combination the operation does not accept).
 * - Values outside the contract (NaN or infinite inputs) produce
 *   unspecified codes; they are never an error.
 */
#ifndef QLINEAR_H
#define QLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QL_OK = 0,
    QL_ERR_VALUE = 1,        /* bad enum value or size                      */
    QL_ERR_DTYPE = 2,        /* unsupported dtype / format combination      */
    QL_ERR_SHAPE = 3,        /* leading dimension smaller than the row      */
    QL_ERR_NULL = 4,         /* a required pointer is NULL                  */
    QL_ERR_UNSUPPORTED = 5,  /* valid request the library does not implement */
    QL_ERR_HIP = 6           /* a HIP runtime call failed                   */
} ql_status;

/* Quantized formats.  E4M3 is OCP E4M3 "fn" (no infinity, NaN 0x7F/0xFF,
 * largest finite 448); E5M2 is OCP E5M2 (largest finite 57344).  The values
 * 0 and 1 are the format numbers of [FP8PY] (_FMT_TO_INT).  INT8 is
 * symmetric, codes in [-127, 127] ([TRACE] step 4).                         */
typedef enum { QL_FMT_E4M3 = 0, QL_FMT_E5M2 = 1, QL_FMT_INT8 = 2 } ql_qfmt;

/* Element types of unquantized tensors (inputs, bias, outputs).            */
typedef enum {
    QL_DT_BF16 = 0,
    QL_DT_FP32 = 1,
    QL_DT_E4M3 = 2,          /* output only: 8-bit E4M3 codes              */
    QL_DT_INT32 = 3          /* output only: raw INT8 x INT8 accumulator   */
} ql_dtype;

/* Scale granularity ([SCMP] "API"): one scale per tensor or one per row.   */
typedef enum { QL_PER_TENSOR = 0, QL_PER_ROW = 1 } ql_gran;

/* Storage of a GEMM operand with logical shape [MN, K]: K_MAJOR stores
 * element (i, k) at p[i*ld + k]; MN_MAJOR stores it at p[k*ld + i].         */
typedef enum { QL_K_MAJOR = 0, QL_MN_MAJOR = 1 } ql_layout;

/* ------------------------------------------------------------------------
 * Workspace
 *
 * Per-tensor amax reductions need a few device words (a running maximum and
 * a counter that elects the last workgroup).  Every call that uses them
 * leaves them reset to zero, so a workspace is zeroed once, at allocation,
 * and never again (the zero-fill dispatch per quantize that [FP8PY]'s commit
 * message removes is not needed at all).  Behind those words the workspace
 * holds scratch that every use overwrites: 1 MiB for grad_bias's partial
 * column sums and 256 KiB for per-workgroup maxima (those of a large
 * quantize's amax pass, which its cast pass reduces, and those of a GEMM of
 * more than 512 workgroups, whose out_amax a one-workgroup kernel reduces
 * after it; smaller GEMM grids elect their last workgroup instead).  Calls
 * that share a workspace must be ordered (same stream or explicit events);
 * concurrent calls need separate workspaces.
 * ---------------------------------------------------------------------- */

/* Size in bytes of one workspace (a constant, 1 KiB + 1.25 MiB). */
size_t ql_workspace_bytes(void);

/* Zero a freshly allocated workspace of `bytes` bytes on `stream` (a fill
 * kernel, no memset node).  Errors: QL_ERR_NULL, QL_ERR_VALUE (too small). */
ql_status ql_workspace_init(void *ws, size_t bytes, void *stream);

/* ------------------------------------------------------------------------
 * ql_quantize -- x_q = sat(RNE(x / scale)) with scale = amax / qmax.
 *
 * [FP8PY] quantize_bf16 (cast with fused amax, amax returned, fresh each
 * call) and _fp8_quantize_cpu (amax = max|x| clamped at 1e-12); [TRACE]
 * steps 2-4 (amax clamped at 1e-8, scale = amax/127, clamp to +-127, round
 * half to even); [SCMP] "API" (per_tensor | per_row).
 *
 *   x        [rows, cols] with leading dimension ldx >= cols; BF16 or FP32.
 *   gran     QL_PER_TENSOR: one amax/scale for the tensor (outputs [1]);
 *            QL_PER_ROW: one per row (outputs [rows]).
 *   fmt      E4M3 (qmax 448), E5M2 (qmax 57344) or INT8 (qmax 127).
 *   scale_in NULL: current scaling, codes use scale = fl32(amax/qmax).
 *            Non-NULL ([1] or [rows]): delayed scaling, codes use *scale_in;
 *            amax is still measured in the same pass.
 *   x_q      [rows, cols] codes, leading dimension ldq >= cols; one byte
 *            per element (FP8 bit pattern, or two's-complement INT8).
 *   scale_out fl32(amax/qmax) of this x ([1] or [rows]); in delayed mode it
 *            is the step a caller would use next.  May be NULL in delayed
 *            mode only.
 *   amax_out max(max|x|, floor), floor = fl32(1e-12) (FP8) or fl32(1e-8)
 *            (INT8) ([1] or [rows]).  May be NULL.
 *   ws       workspace (required for QL_PER_TENSOR, ignored for per-row).
 * Rounding: the quotient is the correctly rounded FP32 x/scale; codes are
 * round-to-nearest-even with saturation to +-qmax; FP8 keeps the sign of a
 * zero result (-0 -> 0x80).  rows == 0 or cols == 0 is a valid no-op except
 * that per-tensor amax/scale are still written (amax = floor).
 * Errors: QL_ERR_NULL, QL_ERR_VALUE (negative size, bad enum), QL_ERR_SHAPE
 * (ldx < cols or ldq < cols), QL_ERR_DTYPE (x_dt not BF16/FP32).
 * ---------------------------------------------------------------------- */
ql_status ql_quantize(const void *x, ql_dtype x_dt, int64_t rows, int64_t cols, int64_t ldx,
                      ql_gran gran, ql_qfmt fmt, const float *scale_in,
                      void *x_q, int64_t ldq, float *scale_out, float *amax_out,
                      void *ws, void *stream);

/* ------------------------------------------------------------------------
 * ql_quantize_ring -- per-tensor delayed scaling with an amax history ring.
 *
 * [FP8PY] linear_forward_fp8 / linear_backward_fp8 docstrings: delayed
 * scaling keeps a float32 buffer with an amax history and the scale, and
 * the quantize kernel itself finalizes it (the measured amax goes to
 * hist[idx], the next step's scale is published on device, no extra
 * launch).  The page packs a counter into the same buffer; here the
 * workspace carries the last-workgroup election, so the ring is
 * [hist | scale].  The page gives no formula for the next scale; this
 * library publishes fl32(fl32(max(hist) / qmax) * 2^margin).
 *
 *   x        [rows, cols], leading dimension ldx >= cols; BF16 or FP32.
 *   fmt      E4M3, E5M2 or INT8.
 *   ring     float32 [hist_len + 1] = [hist | scale], device memory owned
 *            by the caller, read and updated in place.  Initialize the
 *            history to 0 and the scale to a starting step (e.g. 1).
 *   hist_len 1 .. 2^20.  idx: slot of this call's amax, 0 <= idx < hist_len
 *            (the caller advances it, usually modulo hist_len).
 *   margin   -64 .. 64: the published step is scaled by 2^margin.
 *   x_q      [rows, cols] codes (ldq >= cols), cast with the ring's scale
 *            as it was on entry: sat(RNE(x / scale)) as in ql_quantize.
 *   scale_used [1], optional: that scale, for the GEMM that consumes x_q
 *            (the ring's scale has moved on when the call completes).
 *   amax_out [1], optional: max(max|x|, floor) of this x.
 *   ws       workspace (required).
 * One pass over x: 2 bytes (BF16) or 4 read and 1 written per element.
 * Calls that share a ring must be ordered (same stream); they also share
 * the workspace rule of every call.
 * Errors: as ql_quantize, plus QL_ERR_NULL (no ring) and QL_ERR_VALUE
 * (hist_len, idx or margin out of range).
 * ---------------------------------------------------------------------- */
ql_status ql_quantize_ring(const void *x, ql_dtype x_dt, int64_t rows, int64_t cols, int64_t ldx,
                           ql_qfmt fmt, float *ring, int64_t hist_len, int64_t idx, int margin,
                           void *x_q, int64_t ldq, float *scale_used, float *amax_out,
                           void *ws, void *stream);

/* ------------------------------------------------------------------------
 * ql_qgemm -- out = (A_q @ B_q^T) * sa * sb (+ bias), FP32 or INT32
 * accumulation, BF16 / FP32 / E4M3 / INT32 output.
 *
 * [FP8PY] mm_fp8 / fp8_gemm (a @ b * (sa*sb), FP32 accumulation, BF16 or
 * E4M3 output where E4M3 requires out_scale, the output quantization step);
 * linear_forward_fp8 (bias fused into the epilogue); [SCMP] "API" (a @ b.T).
 *
 *   a_q      A [M, K] codes in format a_fmt stored per a_lay with lda.
 *   b_q      B [N, K] codes in format b_fmt stored per b_lay with ldb (the
 *            same bytes as a [K, N] column-major weight).
 *   Formats  FP8 operands may mix E4M3 and E5M2 (backward products pair an
 *            E5M2 gradient with E4M3 weights or activations); INT8 pairs only
 *            with INT8 (else QL_ERR_DTYPE).
 *   sa, sb   FP32 steps: [1] (QL_PER_TENSOR) or [M] / [N] (QL_PER_ROW).
 *   bias     NULL or [N] (BF16 or FP32), added in FP32 after scaling.
 *   out      [M, N] row-major with ldo >= N, element type out_dt:
 *            BF16 / FP32: v = acc*sa*sb + bias, rounded to nearest even;
 *            E4M3: code = sat(RNE(v / *out_scale)) (out_scale required);
 *            INT32 (INT8 operands only): the raw accumulator, no scales or
 *            bias (sa/sb/bias ignored).
 *   out_amax optional [1]: max |v| over all outputs before the output cast
 *            (the next output step of a delayed-scaling caller); needs ws.
 * INT8 accumulation is exact in INT32 for K <= 133144 (K*127^2 < 2^31);
 * larger K is QL_ERR_VALUE.  M, N or K == 0 are valid (K == 0 writes the
 * epilogue of a zero accumulator).
 * Errors: QL_ERR_NULL, QL_ERR_VALUE, QL_ERR_SHAPE (ld too small),
 * QL_ERR_DTYPE (format mix, bias dtype, out dtype vs operands).
 * ---------------------------------------------------------------------- */
ql_status ql_qgemm(const void *a_q, ql_qfmt a_fmt, ql_layout a_lay, int64_t lda,
                   const void *b_q, ql_qfmt b_fmt, ql_layout b_lay, int64_t ldb,
                   int64_t M, int64_t N, int64_t K,
                   const float *sa, ql_gran sa_gran, const float *sb, ql_gran sb_gran,
                   const void *bias, ql_dtype bias_dt,
                   void *out, ql_dtype out_dt, int64_t ldo,
                   const float *out_scale, float *out_amax,
                   void *ws, void *stream);

/* ------------------------------------------------------------------------
 * ql_linear_forward -- quantize x and w per tensor, then the scaled GEMM
 * with the bias fused into its epilogue, all on one stream.
 *
 * [FP8PY] linear_forward_fp8: quantize x and w to fmt, pre-quantized GEMM,
 * bias fused into the epilogue; returns the output, both code tensors and
 * both amax values (here also both steps).
 *
 *   x        [M, K] BF16 or FP32 (x_dt), contiguous.
 *   w        [N, K] same dtype as x, contiguous (nn.Linear weight layout).
 *   bias     NULL or [N] (bias_dt BF16 or FP32).
 *   fmt      E4M3, E5M2 or INT8 for both operands.
 *   sx_in, sw_in  NULL: current scaling; else delayed-scaling steps [1].
 *   out      [M, N] contiguous, out_dt BF16 / FP32 / E4M3 (E4M3 needs
 *            out_scale); out_amax as in ql_qgemm (optional).
 *   x_q [M,K], sx [1], amax_x [1], w_q [N,K], sw [1], amax_w [1]: outputs,
 *            all required.  sx / sw are fl32(amax/qmax) as in ql_quantize:
 *            the steps the GEMM used under current scaling; under delayed
 *            scaling the GEMM uses sx_in / sw_in and sx / sw are the steps a
 *            caller would use next.
 *   ws       workspace (required).
 * Errors: as ql_quantize and ql_qgemm.
 * ---------------------------------------------------------------------- */
ql_status ql_linear_forward(const void *x, ql_dtype x_dt, int64_t M, int64_t K,
                            const void *w, int64_t N,
                            const void *bias, ql_dtype bias_dt, ql_qfmt fmt,
                            const float *sx_in, const float *sw_in,
                            void *out, ql_dtype out_dt, const float *out_scale, float *out_amax,
                            void *x_q, float *sx, float *amax_x,
                            void *w_q, float *sw, float *amax_w,
                            void *ws, void *stream);

/* ------------------------------------------------------------------------
 * ql_linear_forward_noalloc -- ql_linear_forward for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).
 *
 * Arguments, outputs and errors as ql_linear_forward, without `ws`: the
 * workspace is a 1,311,744-byte array inside the library, one copy per
 * GPU, held until the process ends.  Its size does not depend on M, N or
 * K, so every size ql_linear_forward accepts is accepted.  The call makes
 * no device allocation of any kind.  After validation it clears the
 * array's election counters with a small fill kernel on `stream`, then
 * enqueues the same kernels as ql_linear_forward.
 *
 * `stream` (NULL: the default stream) must belong to the current device;
 * otherwise QL_ERR_VALUE.  Every call on one GPU shares that GPU's array:
 * calls that may overlap on one GPU (different streams without ordering
 * between them) race on it and give undefined results.
 * ---------------------------------------------------------------------- */
ql_status ql_linear_forward_noalloc(const void *x, ql_dtype x_dt, int64_t M, int64_t K,
                                    const void *w, int64_t N,
                                    const void *bias, ql_dtype bias_dt, ql_qfmt fmt,
                                    const float *sx_in, const float *sw_in,
                                    void *out, ql_dtype out_dt, const float *out_scale, float *out_amax,
                                    void *x_q, float *sx, float *amax_x,
                                    void *w_q, float *sw, float *amax_w, void *stream);

/* ------------------------------------------------------------------------
 * ql_quantize_groups -- one scale per group of rows.
 *
 * [SCMP] "API": group_a / group_b set the row-group size of an operand's
 * scales, and granularity per_head quantizes a (BH, N, D) operand one head
 * at a time.  Both are row groups of the flattened matrix: group_rows = 1
 * is per-row, = rows per-tensor, = N per head of [BH*N, D].
 *
 *   x, x_dt, rows, cols, ldx, fmt, x_q, ldq: as ql_quantize.
 *   group_rows >= 1: rows [g*G, min((g+1)*G, rows)) share scale g.
 *   scale_in NULL (current scaling) or [ngroups] delayed steps.
 *   scale_out, amax_out [ngroups], ngroups = ceil(rows / G): as ql_quantize
 *            per group (scale_out may be NULL only with scale_in).
 * One workgroup per group: meant for groups of up to a few hundred
 * thousand elements (heads, row groups); use ql_quantize for a whole large
 * tensor.  No workspace is needed.
 * Errors: as ql_quantize, plus QL_ERR_VALUE for group_rows < 1.
 * ---------------------------------------------------------------------- */
ql_status ql_quantize_groups(const void *x, ql_dtype x_dt, int64_t rows, int64_t cols, int64_t ldx,
                             int64_t group_rows, ql_qfmt fmt, const float *scale_in,
                             void *x_q, int64_t ldq, float *scale_out, float *amax_out, void *stream);

/* ------------------------------------------------------------------------
 * ql_qgemm_batched -- batched scaled GEMM with row-group scales.
 *
 * [SCMP] "API" (per_head: (BH, N, D) operands, N != M allowed; group_a /
 * group_b): out[z] = (A[z] . B[z]^T) * sa * sb (+ bias) for z < batch, each
 * item exactly as ql_qgemm (layouts, formats, epilogue, outputs).
 *
 *   a_q + z*stride_a, b_q + z*stride_b: item z's operands (strides in
 *            elements = bytes); out + z*stride_out (elements of out_dt).
 *   batch    1 .. 65535.
 *   sa, group_a: scale of A row m of item z is sa[(z*M + m) / group_a]
 *            (row groups over the flattened batch; group_a = M gives one
 *            scale per item, i.e. per head; 0 = one scale sa[0] for all).
 *            sa holds ceil(batch*M / group_a) floats (1 when group_a is
 *            0); sb, group_b likewise with z*N + n.
 *   bias [N] shared by all items; out_amax covers every item.
 * Operand items may overlap; output items must not.  Strides that are not
 * multiples of 16 bytes are accepted and take the unaligned (slower)
 * staging.  Items take the general kernel (the pipelined one serves
 * batch == 1).
 * Errors: as ql_qgemm, plus QL_ERR_VALUE for batch, group or stride out of
 * range.
 * ---------------------------------------------------------------------- */
ql_status ql_qgemm_batched(const void *a_q, ql_qfmt a_fmt, ql_layout a_lay, int64_t lda, int64_t stride_a,
                           const void *b_q, ql_qfmt b_fmt, ql_layout b_lay, int64_t ldb, int64_t stride_b,
                           int64_t batch, int64_t M, int64_t N, int64_t K,
                           const float *sa, int64_t group_a, const float *sb, int64_t group_b,
                           const void *bias, ql_dtype bias_dt,
                           void *out, ql_dtype out_dt, int64_t ldo, int64_t stride_out,
                           const float *out_scale, float *out_amax, void *ws, void *stream);

/* ------------------------------------------------------------------------
 * ql_linear_forward_static -- static FP8 inference.
 *
 * [FP8PY] linear_forward_fp8 docstring: for static inference the weight
 * (and optionally the bias) arrive already quantized to the layer's format,
 * with their steps; a quantized bias needs its own step (bias_scale) and
 * the weight's amax is not measured.  Only x is quantized here:
 *   x_q = quantize(x) (per tensor, current or delayed as sx_in says),
 *   out = (x_q . w_q^T) * sx * sw + bias.
 *
 *   x, x_dt, M, K, sx_in, x_q, sx, amax_x, out, out_dt, out_scale, out_amax,
 *            ws: as ql_linear_forward.
 *   w_q      [N, K] codes of `fmt` (leading dimension K); sw its step [1].
 *   fmt      E4M3 or E5M2.
 *   bias     NULL; or [N] BF16/FP32 values (bias_dt) with bias_scale NULL;
 *            or, with bias_scale non-NULL ([1]), [N] codes of `fmt` whose
 *            values are dec(code) * bias_scale (bias_dt is then ignored).
 * Errors: as ql_linear_forward; QL_ERR_DTYPE for INT8; QL_ERR_NULL without
 * sw.
 * ---------------------------------------------------------------------- */
ql_status ql_linear_forward_static(const void *x, ql_dtype x_dt, int64_t M, int64_t K,
                                  const void *w_q, int64_t N, const float *sw,
                                  const void *bias, ql_dtype bias_dt, const float *bias_scale,
                                  ql_qfmt fmt, const float *sx_in,
                                  void *out, ql_dtype out_dt, const float *out_scale, float *out_amax,
                                  void *x_q, float *sx, float *amax_x, void *ws, void *stream);

/* ------------------------------------------------------------------------
 * ql_linear_backward -- backward of the quantized linear layer.
 *
 * [FP8PY] linear_backward_fp8 docstring: the output gradient is quantized
 * once (E5M2 by default, the wider range) and that quantization is shared
 * by the two matrix-core products; grad_bias comes back beside them and
 * `masks` selects which results are produced.  The products take the
 * forward's codes (the backward workload pairs an E5M2 gradient with the
 * E4M3 forward operands) in their stored layouts, with no transposed
 * copies:
 *   dX [M, K] = (g_q . W) * sg * sw   (W read MN-major from w_q [N, K])
 *   dW [N, K] = (g_q^T . X) * sg * sx (g_q and x_q [M, K] read MN-major)
 *   dbias [N] = column sums of the BF16 g (FP32; the summation order
 *            depends on M and N only, so results repeat bit for bit)
 *
 *   g        BF16 [M, N] row-major (leading dimension N).
 *   x_q, sx  forward codes of x [M, K] (leading dimension K) and their
 *            per-tensor step [1]; w_q, sw the same for w [N, K].
 *   masks    non-empty OR of QL_BWD_DX, QL_BWD_DW, QL_BWD_DBIAS.
 *   g_fmt    E4M3 or E5M2 (x_fmt / w_fmt likewise; INT8 is not a backward
 *            format).  sg_in: NULL = current scaling (sg = amax/qmax of
 *            g), else the delayed step [1] the codes use.
 *   dx, dw   outputs ([M, K], [N, K], leading dimension K) in out_dt (BF16
 *            or FP32); required when their mask bit is set.
 *   dbias    FP32 [N], required with QL_BWD_DBIAS.
 *   g_q, sg, amax_g  g's codes [M, N] and its per-tensor step and amax, as
 *            ql_quantize writes them; required when dX or dW is produced.
 *   ws       workspace (required).
 * Errors: as ql_quantize and ql_qgemm, plus QL_ERR_VALUE for a bad mask.
 * ---------------------------------------------------------------------- */
#define QL_BWD_DX 1u
#define QL_BWD_DW 2u
#define QL_BWD_DBIAS 4u
ql_status ql_linear_backward(const void *g, int64_t M, int64_t N,
                             const void *x_q, ql_qfmt x_fmt, const float *sx,
                             const void *w_q, ql_qfmt w_fmt, const float *sw, int64_t K,
                             unsigned masks, ql_qfmt g_fmt, const float *sg_in,
                             void *dx, void *dw, ql_dtype out_dt, float *dbias,
                             void *g_q, float *sg, float *amax_g, void *ws, void *stream);

/* Short fixed text for a status code (never NULL). */
const char *ql_status_string(ql_status s);

/* Detail of the last error on the calling thread ("" if none). */
const char *ql_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* QLINEAR_H */
