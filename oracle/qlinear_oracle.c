/*
 * qlinear_oracle.c -- plain, slow CPU oracle for the absmax-scaled quantized
 * linear layer (quantize -> scaled low-precision GEMM -> epilogue).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant with the HIP library and must never be used as a
 * fallback for it.
 *
 * Sources (web pages; cited by title and section):
 *   [FP8PY]  AstrAI, astrai/extension/ops/fp8.py at commit 5e76fbd -- module
 *            docstring (scale semantics), _fp8_quantize_cpu, fp8_gemm /
 *            _fp8_gemm_cpu, mm_fp8 and linear_forward_fp8 docstrings.
 *   [TRACE]  POPCORNBENCH page "Kimi-K2.6 l2_p13" -- the reference model's
 *            steps 2-4 (symmetric INT8 fake-quant) and the discussion of
 *            round-half-to-even (nearbyintf vs roundf).
 *   [SCMP]   CrucibleComputingGroup/scmp_kernels README -- "SC quickstart" and
 *            "API" (per_tensor / per_row granularity, a @ b.T orientation).
 *
 * Every floating-point step is done in IEEE double unless a page fixes the
 * precision.  Two places are fixed to FP32 by the pages: the quantization step
 * itself (scale = amax/qmax as an FP32 tensor op) and the quotient x/scale
 * ([FP8PY] _fp8_quantize_cpu divides x.float() by the FP32 scale; [TRACE]
 * divides the FP32 input by the FP32 scale).  Both are formed as the double
 * quotient and then rounded once to float.  For operands of p = 24 bits, a
 * quotient rounded first to q = 53 >= 2p + 2 bits and then to p bits equals
 * the directly rounded quotient (Figueroa, "When is double rounding
 * innocuous?", SIGNUM 1995), so this is the correctly rounded FP32 division.
 *
 * Build: gcc -std=c11 -O2 -fPIC -shared -ffp-contract=off (no -ffast-math).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* Format and dtype numbers used by this file's entry points. */
enum { ORC_E4M3 = 0, ORC_E5M2 = 1, ORC_INT8 = 2 };
enum { ORC_IN_BF16 = 0, ORC_IN_FP32 = 1, ORC_BIAS_F64 = 2 };
enum { ORC_PER_TENSOR = 0, ORC_PER_ROW = 1 };
enum { ORC_K_MAJOR = 0, ORC_MN_MAJOR = 1 };

/* ------------------------------------------------------------------------ */
/* Format parameters (OCP 8-bit floating point: E4M3 "fn" has no infinity and
 * one NaN pattern per sign, 0x7F/0xFF; E5M2 keeps IEEE-style inf/NaN).
 * [FP8PY] _fmt_dtype maps "e4m3" to torch.float8_e4m3fn, "e5m2" to
 * torch.float8_e5m2.                                                        */
typedef struct {
    int mbits;     /* stored mantissa bits                                  */
    int bias;      /* exponent bias                                         */
    int emin;      /* exponent of the smallest normal                       */
    double maxv;   /* largest finite magnitude                              */
    int maxcode;   /* code (sign bit clear) of the largest finite magnitude */
} orc_fp8_spec;

static orc_fp8_spec orc_spec(int fmt)
{
    orc_fp8_spec s;
    if (fmt == ORC_E4M3) {
        s.mbits = 3; s.bias = 7; s.emin = -6; s.maxv = 448.0; s.maxcode = 0x7E;
    } else {
        s.mbits = 2; s.bias = 15; s.emin = -14; s.maxv = 57344.0; s.maxcode = 0x7B;
    }
    return s;
}

/* Largest magnitude of the quantized format: qmax in scale = amax / qmax. */
double orc_qmax(int fmt)
{
    if (fmt == ORC_INT8) return 127.0;         /* [TRACE] step 3: amax/127 */
    return orc_spec(fmt).maxv;
}

/* Floor applied to amax before the scale is formed.  [FP8PY]
 * _fp8_quantize_cpu clamps amax at 1e-12; [TRACE] step 2 clamps at 1e-8 for
 * the INT8 fake-quant.  Both clamps act on FP32 tensors, so the floors are
 * the FP32 values nearest to those decimals.                               */
float orc_amax_floor(int fmt)
{
    return fmt == ORC_INT8 ? (float)1e-8 : (float)1e-12;
}

/* Round half to even of a double, written out so that it does not depend on
 * the floating-point environment.  [TRACE] round-half-to-even discussion:
 * torch.round sends ties to the even neighbour.                             */
static double orc_rne(double n)
{
    double f = floor(n);
    double d = n - f;                  /* exact for |n| < 2^52 */
    if (d > 0.5) return f + 1.0;
    if (d < 0.5) return f;
    return fmod(f, 2.0) == 0.0 ? f : f + 1.0;
}

/* ------------------------------------------------------------------------ */
/* FP8 encode: round to nearest even, saturate to +-max, keep the sign of 0.
 * v is the (FP32) quotient x/scale, passed as a double.                     */
int orc_fp8_encode(double v, int fmt)
{
    orc_fp8_spec s = orc_spec(fmt);
    int sign = signbit(v) ? 0x80 : 0;
    double a = fabs(v);
    if (isnan(v)) return sign | 0x7F;
    if (a >= s.maxv) return sign | s.maxcode;        /* saturation */
    if (a == 0.0) return sign;                        /* -0 -> 0x80 */
    int ex;
    (void)frexp(a, &ex);                              /* a = f*2^ex, f in [0.5,1) */
    int e = ex - 1;                                   /* floor(log2 a) */
    if (e < s.emin) e = s.emin;                       /* subnormal binade */
    double n = ldexp(a, s.mbits - e);                 /* exact scaling */
    double r = orc_rne(n);
    int one = 1 << s.mbits;
    if (r == (double)(2 * one)) { r = (double)one; e += 1; }
    int ir = (int)r;
    int efield = ir < one ? 0 : e + s.bias;
    int mant = ir < one ? ir : ir - one;
    return sign | (efield << s.mbits) | mant;
}

/* FP8 decode: exact.  E4M3: field 0 -> m*2^-9, else (1+m/8)*2^(E-7);
 * 0x7F/0xFF are NaN.  E5M2: field 0 -> m*2^-16, field 31 -> inf/NaN,
 * else (1+m/4)*2^(E-15).                                                    */
double orc_fp8_decode(int code, int fmt)
{
    orc_fp8_spec s = orc_spec(fmt);
    int sign = (code >> 7) & 1;
    int efield = (code >> s.mbits) & ((1 << (7 - s.mbits)) - 1);
    int mant = code & ((1 << s.mbits) - 1);
    int emax_field = (1 << (7 - s.mbits)) - 1;
    double v;
    if (fmt == ORC_E4M3 && efield == emax_field && mant == 7) {
        v = NAN;
    } else if (fmt == ORC_E5M2 && efield == emax_field) {
        v = mant == 0 ? INFINITY : NAN;
    } else if (efield == 0) {
        v = ldexp((double)mant, s.emin - s.mbits);
    } else {
        v = ldexp((double)((1 << s.mbits) + mant), efield - s.bias - s.mbits);
    }
    return sign ? -v : v;
}

/* Symmetric INT8 encode: clamp(round_half_even(v), -127, 127).  [TRACE]
 * step 4; -128 is never produced.  A NaN quotient is out of contract and
 * maps to 0.                                                                */
int orc_int8_encode(double v)
{
    if (isnan(v)) return 0;
    double r;
    if (v >= 127.0) r = 127.0;
    else if (v <= -127.0) r = -127.0;
    else r = orc_rne(v);
    return (int)r;
}

/* ------------------------------------------------------------------------ */
/* Inputs: BF16 is the top half of an FP32 word (exact decode); FP32 as is.  */
static double orc_load(const void *x, int dt, int64_t idx)
{
    if (dt == ORC_IN_BF16) {
        uint32_t u = (uint32_t)((const uint16_t *)x)[idx] << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        return (double)f;
    }
    return (double)((const float *)x)[idx];
}

/* Correctly rounded FP32 quotient (see the header note on double rounding). */
float orc_div_f32(float x, float s)
{
    return (float)((double)x / (double)s);
}

/* amax = max |x| over the tensor (out[0]) or over each row (out[r]),
 * before any floor.  Exact and independent of the reduction order.         */
void orc_amax_raw(const void *x, int dt, int64_t rows, int64_t cols, int64_t ldx,
                  int gran, double *out)
{
    int64_t nout = gran == ORC_PER_ROW ? rows : 1;
    for (int64_t i = 0; i < nout; ++i) out[i] = 0.0;
    for (int64_t r = 0; r < rows; ++r) {
        double *dst = gran == ORC_PER_ROW ? &out[r] : &out[0];
        for (int64_t c = 0; c < cols; ++c) {
            double a = fabs(orc_load(x, dt, r * ldx + c));
            if (a > *dst || isnan(a)) *dst = a;
        }
    }
}

/* Quantize, following the steps of [FP8PY] (quantize_bf16 docstring and
 * _fp8_quantize_cpu) and [TRACE] (steps 2-4):
 *   1. amax = max(max|x|, floor)              (per tensor or per row)
 *   2. scale = fl32(amax / qmax)              (current scaling), or the given
 *      scale_in (delayed scaling: the step is an input, amax still measured)
 *   3. v = fl32(x / scale)
 *   4. code = sat(RNE(v)) in the target format
 * scale_out receives fl32(amax/qmax) in both modes; amax_out the floored
 * amax.  Granularity: one scale for the whole tensor, or one per row
 * ([SCMP] "API": per_tensor | per_row).                                     */
void orc_quantize(const void *x, int dt, int64_t rows, int64_t cols, int64_t ldx,
                  int gran, int fmt, const float *scale_in,
                  uint8_t *xq, int64_t ldq, float *scale_out, float *amax_out)
{
    int64_t nout = gran == ORC_PER_ROW ? rows : 1;
    float floor_f = orc_amax_floor(fmt);
    double qmax = orc_qmax(fmt);
    /* step 1, then step 2, for each scale group (the tensor, or one row) */
    for (int64_t i = 0; i < nout; ++i) {
        double m = 0.0;
        int64_t r0 = gran == ORC_PER_ROW ? i : 0;
        int64_t r1 = gran == ORC_PER_ROW ? i + 1 : rows;
        for (int64_t r = r0; r < r1; ++r)
            for (int64_t c = 0; c < cols; ++c) {
                double a = fabs(orc_load(x, dt, r * ldx + c));
                if (a > m || isnan(a)) m = a;
            }
        float amax = (float)m;                 /* exact: m is an input magnitude */
        if (!(amax >= floor_f) && !isnan(amax)) amax = floor_f;
        amax_out[i] = amax;
        /* step 2 */
        scale_out[i] = (float)((double)amax / qmax);
    }
    /* steps 3-4 */
    for (int64_t r = 0; r < rows; ++r) {
        int64_t g = gran == ORC_PER_ROW ? r : 0;
        float scale = scale_in ? scale_in[g] : scale_out[g];
        for (int64_t c = 0; c < cols; ++c) {
            float xv = (float)orc_load(x, dt, r * ldx + c);
            float v = orc_div_f32(xv, scale);
            int code = fmt == ORC_INT8 ? (orc_int8_encode((double)v) & 0xFF)
                                       : orc_fp8_encode((double)v, fmt);
            xq[r * ldq + c] = (uint8_t)code;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Row-group quantization ([SCMP] "API": group_a / group_b, the row-group
 * size of an operand's scales; per_head on a (BH, N, D) tensor is one scale
 * per N consecutive rows of the flattened [BH*N, D]).  One scale per group
 * of group_rows consecutive rows (the last group may be shorter); within a
 * group, steps 1-4 exactly as for a tensor.                                */
void orc_quantize_groups(const void *x, int dt, int64_t rows, int64_t cols, int64_t ldx,
                         int64_t group_rows, int fmt, const float *scale_in,
                         uint8_t *xq, int64_t ldq, float *scale_out, float *amax_out)
{
    int64_t ngroups = rows == 0 ? 0 : (rows + group_rows - 1) / group_rows;
    float floor_f = orc_amax_floor(fmt);
    double qmax = orc_qmax(fmt);
    for (int64_t g = 0; g < ngroups; ++g) {
        int64_t r0 = g * group_rows, r1 = r0 + group_rows < rows ? r0 + group_rows : rows;
        double m = 0.0;
        for (int64_t r = r0; r < r1; ++r)
            for (int64_t c = 0; c < cols; ++c) {
                double a = fabs(orc_load(x, dt, r * ldx + c));
                if (a > m || isnan(a)) m = a;
            }
        float amax = (float)m;
        if (!(amax >= floor_f) && !isnan(amax)) amax = floor_f;
        amax_out[g] = amax;
        scale_out[g] = (float)((double)amax / qmax);
        float scale = scale_in ? scale_in[g] : scale_out[g];
        for (int64_t r = r0; r < r1; ++r)
            for (int64_t c = 0; c < cols; ++c) {
                float v = orc_div_f32((float)orc_load(x, dt, r * ldx + c), scale);
                int code = fmt == ORC_INT8 ? (orc_int8_encode((double)v) & 0xFF) : orc_fp8_encode((double)v, fmt);
                xq[r * ldq + c] = (uint8_t)code;
            }
    }
}

/* ------------------------------------------------------------------------ */
/* Delayed-scaling amax history ("scale ring").  [FP8PY] linear_forward_fp8
 * and linear_backward_fp8 docstrings: the ring is a float32 buffer holding
 * an amax history and the scale; the quantize of step t casts with the
 * scale already in the ring (delayed scaling), stores the amax it measures
 * at hist[idx], and publishes the scale for the next step.  The page gives
 * no formula for that scale; the reading taken here (the usual delayed
 * scaling rule) is
 *     next = fl32( fl32(max_i hist[i] / qmax) * 2^margin )
 * with the measured amax floored as in current scaling, so an all-zero
 * history still gives a positive step.  ring = [hist (hist_len) | scale].
 * This function does the bookkeeping after the cast; the cast itself is
 * orc_quantize with scale_in = the ring's old scale.                       */
void orc_ring_update(float *ring, int64_t hist_len, int64_t idx, int margin, int fmt, float amax)
{
    double qmax = orc_qmax(fmt);
    ring[idx] = amax;
    double m = 0.0;
    for (int64_t i = 0; i < hist_len; ++i)
        if ((double)ring[i] > m) m = ring[i];
    float step = (float)(m / qmax);
    ring[hist_len] = (float)ldexp((double)step, margin);
}

/* ------------------------------------------------------------------------ */
/* GEMM.  C[m,n] = sum_k dec(A[m,k]) * dec(B[n,k])  ([SCMP] "API": a @ b.T;
 * [FP8PY] fp8_gemm: FP32 accumulation of a @ b).  A is [M,K], B is [N,K];
 * K-major means k is the contiguous index (A[m*lda+k]), MN-major means m (or
 * n) is (A[k*lda+m]).
 *
 * The oracle forms the sum exactly: every E4M3 value is an integer multiple
 * of 2^-9, every E5M2 value a multiple of 2^-16, every INT8 value an integer,
 * so the products are integers times 2^-(fa+fb) and the sum is an exact
 * 128-bit integer.  It also returns S = sum_k |dec(A)*dec(B)| (exact, used by
 * the error bound on floating-point outputs) and, for INT8, the integer sum.
 * Codes that decode to NaN or infinity are out of contract: the entry is
 * then reported as NaN.
 *
 * Optionally (hbound_out != NULL) it also returns H, an upper bound on the
 * error of a matrix core that sums each aligned group of `group` consecutive
 * products (k = 0..group-1, group..2*group-1, ...) by aligning every product
 * to the group's largest operand-exponent sum e_a + e_b and truncating it
 * toward zero after `fbits` fraction bits: every product that is not a
 * multiple of 2^(max(e_a+e_b) - fbits) adds that grid step to H.  H is not
 * part of the reference value; it only feeds the acceptance bound of
 * floating-point GEMM outputs (the measured FP8 matrix-core behaviour is
 * group = 8, fbits = 13).  INT8 products are integers and contribute 0.    */
static int orc_frac_bits(int fmt)
{
    return fmt == ORC_E4M3 ? 9 : fmt == ORC_E5M2 ? 16 : 0;
}

/* Decoded value times 2^frac_bits, as an integer; returns 0 on NaN/inf.    */
static int orc_fixed(int code, int fmt, int64_t *out)
{
    if (fmt == ORC_INT8) { *out = (int64_t)(int8_t)code; return 1; }
    double v = orc_fp8_decode(code, fmt);
    if (!isfinite(v)) return 0;
    *out = (int64_t)ldexp(v, orc_frac_bits(fmt));     /* exact integer */
    return 1;
}

static uint8_t orc_elem(const uint8_t *p, int lay, int64_t ld, int64_t mn, int64_t k)
{
    return lay == ORC_K_MAJOR ? p[mn * ld + k] : p[k * ld + mn];
}

/* Unbiased exponent of an FP8 operand as the alignment logic sees it
 * (subnormals and zero at the minimum normal exponent).                    */
static int orc_operand_exp(int code, int fmt)
{
    orc_fp8_spec s = orc_spec(fmt);
    int efield = (code >> s.mbits) & ((1 << (7 - s.mbits)) - 1);
    return efield == 0 ? s.emin : efield - s.bias;
}

void orc_qgemm_entries(const uint8_t *a, int a_fmt, int a_lay, int64_t lda,
                       const uint8_t *b, int b_fmt, int b_lay, int64_t ldb,
                       int64_t K, const int64_t *ms, const int64_t *ns, int64_t count,
                       double *acc_out, double *abs_out, int64_t *iacc_out,
                       double *hbound_out, int group, int fbits)
{
    int shift = orc_frac_bits(a_fmt) + orc_frac_bits(b_fmt);
    int is_int = a_fmt == ORC_INT8 && b_fmt == ORC_INT8;
    for (int64_t e = 0; e < count; ++e) {
        __int128 sum = 0, sabs = 0;
        double hb = 0.0;
        int finite = 1;
        for (int64_t k0 = 0; k0 < K; k0 += group > 0 ? group : K) {
            int64_t k1 = group > 0 && k0 + group < K ? k0 + group : K;
            int emax = -100000;
            for (int64_t k = k0; k < k1; ++k) {
                int64_t ia, ib;
                uint8_t ca = orc_elem(a, a_lay, lda, ms[e], k);
                uint8_t cb = orc_elem(b, b_lay, ldb, ns[e], k);
                int ok_a = orc_fixed(ca, a_fmt, &ia);
                int ok_b = orc_fixed(cb, b_fmt, &ib);
                if (!ok_a || !ok_b) { finite = 0; continue; }
                __int128 p = (__int128)ia * (__int128)ib;
                sum += p;
                sabs += p < 0 ? -p : p;
                if (!is_int && p != 0) {
                    int es = orc_operand_exp(ca, a_fmt) + orc_operand_exp(cb, b_fmt);
                    if (es > emax) emax = es;
                }
            }
            if (hbound_out && !is_int && emax > -100000) {
                double grid = ldexp(1.0, emax - fbits);
                for (int64_t k = k0; k < k1; ++k) {
                    double pa = orc_fp8_decode(orc_elem(a, a_lay, lda, ms[e], k), a_fmt);
                    double pb = orc_fp8_decode(orc_elem(b, b_lay, ldb, ns[e], k), b_fmt);
                    double p = fabs(pa * pb);            /* exact: <= 8 significant bits */
                    if (p != 0.0 && fmod(p, grid) != 0.0) hb += grid;
                }
            }
        }
        if (!finite) {
            acc_out[e] = NAN; abs_out[e] = NAN;
            if (iacc_out) iacc_out[e] = 0;
            if (hbound_out) hbound_out[e] = NAN;
            continue;
        }
        acc_out[e] = ldexp((double)sum, -shift);
        abs_out[e] = ldexp((double)sabs, -shift);
        if (iacc_out) iacc_out[e] = (int64_t)sum;
        if (hbound_out) hbound_out[e] = hb;
    }
}

/* Epilogue reference value, in double from the exact accumulator:
 *   v = acc * sa * sb + bias
 * ([FP8PY] fp8_gemm docstring: a @ b * (sa * sb); linear_forward_fp8
 * docstring: the bias is fused into the GEMM epilogue).  sa/sb are indexed
 * per row of A / per row of B when their granularity is per-row, else [0].
 * bias may be NULL (no bias); bias_dt is 0 = BF16 bits, 1 = FP32.          */
void orc_epilogue(const double *acc, const int64_t *ms, const int64_t *ns, int64_t count,
                  const float *sa, int sa_gran, const float *sb, int sb_gran,
                  const void *bias, int bias_dt, double *v_out)
{
    for (int64_t e = 0; e < count; ++e) {
        double v = acc[e] * (double)sa[sa_gran == ORC_PER_ROW ? ms[e] : 0]
                          * (double)sb[sb_gran == ORC_PER_ROW ? ns[e] : 0];
        if (bias) v += bias_dt == ORC_BIAS_F64 ? ((const double *)bias)[ns[e]] : orc_load(bias, bias_dt, ns[e]);
        v_out[e] = v;
    }
}

/* Static FP8 inference ([FP8PY] linear_forward_fp8 docstring): the bias may
 * arrive quantized to the layer's format with its own step bias_scale; its
 * value is then dec(code) * bias_scale (exact in double).                  */
void orc_qbias_values(const uint8_t *codes, int64_t n, int fmt, float bias_scale, double *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_fp8_decode(codes[i], fmt) * (double)bias_scale;
}

/* FP8 output: code = sat(RNE(v / out_scale)) in E4M3.  out_scale is the
 * output quantization step ([FP8PY] fp8_gemm / mm_fp8 docstrings: the value
 * divided out when quantizing).                                             */
void orc_fp8_output(const double *v, int64_t count, float out_scale, int fmt,
                    uint8_t *codes)
{
    for (int64_t e = 0; e < count; ++e)
        codes[e] = (uint8_t)orc_fp8_encode(v[e] / (double)out_scale, fmt);
}
