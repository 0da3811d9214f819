// qlinear_api.cpp -- the C ABI declared in include/qlinear.h.
//
// Every entry point validates all arguments on the host first and enqueues
// nothing when any check fails, mirroring the raise-before-launch checks of
// AstrAI ops/fp8.py @5e76fbd (_fmt_int raises ValueError for an unknown
// format; the cuda kernels raise TypeError for a wrong dtype; mm_fp8 raises
// ValueError for an unknown out_dtype).  Then it picks a kernel instance by
// format, layout and alignment and launches on the caller's stream.
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdint>
#include <string>

#include "internal.hpp"
#include "qdev.hpp"
#include "qlinear.h"

namespace ql {
hipError_t launch_qgemm_e4m3_e4m3(const GemmParams &p, int a_mn, int b_mn, hipStream_t s);
hipError_t launch_qgemm_e4m3_e5m2(const GemmParams &p, int a_mn, int b_mn, hipStream_t s);
hipError_t launch_qgemm_e5m2_e4m3(const GemmParams &p, int a_mn, int b_mn, hipStream_t s);
hipError_t launch_qgemm_e5m2_e5m2(const GemmParams &p, int a_mn, int b_mn, hipStream_t s);
hipError_t launch_qgemm_int8_int8(const GemmParams &p, int a_mn, int b_mn, hipStream_t s);

hipError_t launch_qgemm(const GemmParams &pp, int a_fmt, int b_fmt, int a_mn, int b_mn, hipStream_t s)
{
    GemmParams p = pp;
    finish_groups(p);
    if (a_fmt == FMT_INT8) return launch_qgemm_int8_int8(p, a_mn, b_mn, s);
    if (a_fmt == FMT_E4M3) return b_fmt == FMT_E4M3 ? launch_qgemm_e4m3_e4m3(p, a_mn, b_mn, s)
                                                    : launch_qgemm_e4m3_e5m2(p, a_mn, b_mn, s);
    return b_fmt == FMT_E4M3 ? launch_qgemm_e5m2_e4m3(p, a_mn, b_mn, s)
                             : launch_qgemm_e5m2_e5m2(p, a_mn, b_mn, s);
}

int device_cu_count()
{
    constexpr int MAX_DEV = 64;
    static std::atomic<int> cache[MAX_DEV];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEV) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}
}  // namespace ql

namespace {

thread_local std::string g_last_error;

ql_status fail(ql_status st, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

ql_status ok()
{
    g_last_error.clear();
    return QL_OK;
}

ql_status hip_status(hipError_t e, const char *what)
{
    if (e == hipSuccess) return ok();
    return fail(QL_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t INT8_K_MAX = 133144;          // K * 127^2 <= 2^31 - 1
constexpr int64_t MAX_DIM = (int64_t)1 << 40;   // keeps every byte offset far inside int64
constexpr int64_t RING_MAX_HIST = (int64_t)1 << 20;
constexpr int RING_MAX_MARGIN = 64;

bool valid_fmt(int f) { return f == QL_FMT_E4M3 || f == QL_FMT_E5M2 || f == QL_FMT_INT8; }
bool valid_gran(int g) { return g == QL_PER_TENSOR || g == QL_PER_ROW; }
bool valid_layout(int l) { return l == QL_K_MAJOR || l == QL_MN_MAJOR; }
bool valid_dtype(int d) { return d >= QL_DT_BF16 && d <= QL_DT_INT32; }

float fmt_qmax(int fmt) { return fmt == QL_FMT_E4M3 ? 448.0f : fmt == QL_FMT_E5M2 ? 57344.0f : 127.0f; }
float fmt_floor(int fmt) { return fmt == QL_FMT_INT8 ? 1e-8f : 1e-12f; }

// ---------------------------------------------------------------------------
ql_status check_quantize(const void *x, int x_dt, int64_t rows, int64_t cols, int64_t ldx, int gran,
                         int fmt, const float *scale_in, const void *x_q, int64_t ldq,
                         const float *scale_out, const void *ws)
{
    if (!valid_dtype(x_dt)) return fail(QL_ERR_VALUE, "quantize: unknown input dtype %d", x_dt);
    if (x_dt != QL_DT_BF16 && x_dt != QL_DT_FP32)
        return fail(QL_ERR_DTYPE, "quantize requires BF16 or FP32 input, got dtype %d", x_dt);
    if (!valid_gran(gran)) return fail(QL_ERR_VALUE, "quantize: unknown granularity %d", gran);
    if (!valid_fmt(fmt)) return fail(QL_ERR_VALUE, "quantize: unsupported format %d (expected 0=e4m3, 1=e5m2, 2=int8)", fmt);
    if (rows < 0 || cols < 0) return fail(QL_ERR_VALUE, "quantize: negative size rows=%lld cols=%lld",
                                          (long long)rows, (long long)cols);
    if (rows > MAX_DIM || cols > MAX_DIM) return fail(QL_ERR_VALUE, "quantize: size too large");
    if (rows > 0 && (ldx < cols || ldq < cols))
        return fail(QL_ERR_SHAPE, "quantize: leading dimensions ldx=%lld ldq=%lld must be >= cols=%lld",
                    (long long)ldx, (long long)ldq, (long long)cols);
    if (rows > 0 && cols > 0 && (!x || !x_q)) return fail(QL_ERR_NULL, "quantize: x and x_q are required");
    if (!scale_in && !scale_out && (gran == QL_PER_TENSOR || rows > 0))
        return fail(QL_ERR_NULL, "quantize: scale_out is required under current scaling");
    if (gran == QL_PER_TENSOR && !ws) return fail(QL_ERR_NULL, "quantize: per-tensor quantize needs a workspace");
    if (gran == QL_PER_ROW && rows > 0x7FFFFFFF)
        return fail(QL_ERR_UNSUPPORTED, "quantize: per-row quantize supports at most 2^31-1 rows");
    return QL_OK;
}

// ws: the caller's workspace (NULL for per-row); slot: this tensor's counter
// slot and block of per-workgroup maxima in it.
ql::QzParams make_qz(const void *x, int x_dt, int64_t rows, int64_t cols, int64_t ldx, int gran, int fmt,
                     const float *scale_in, void *x_q, int64_t ldq, float *scale_out, float *amax_out,
                     void *ws, int64_t slot)
{
    ql::QzParams p{};
    p.x = x; p.rows = rows; p.cols = cols; p.ldx = ldx;
    p.xq = x_q; p.ldq = ldq;
    p.scale_out = scale_out; p.amax_out = amax_out;
    p.scale_src = scale_in ? scale_in : scale_out;
    p.ws = ws ? ql::ws_slot(ws, slot) : nullptr;
    p.amax_part = ws && gran == QL_PER_TENSOR ? ql::ws_amax_parts(ws) + slot * ql::QZ_PARTS_PER_SLOT : nullptr;
    p.qmax = fmt_qmax(fmt);
    p.floor = fmt_floor(fmt);
    p.n_elems = rows * cols;
    p.per_row = gran == QL_PER_ROW;
    p.group_rows = 1;
    p.delayed = scale_in != nullptr;
    const bool al = aligned16(x) && aligned16(x_q);
    const bool flat = (ldx == cols && ldq == cols) || rows <= 1;
    const bool rowvec = cols % 16 == 0 && ldx % 16 == 0 && ldq % 16 == 0;
    if (flat && al) {
        p.mode = 0;
        p.n_units = p.n_elems / 16;
    } else if (rowvec && al) {
        p.mode = 1;
        p.units_per_row = cols / 16;
        p.n_units = rows * p.units_per_row;
    } else {
        p.mode = 2;
    }
    p.vec_rows = rowvec && al;
    if (p.per_row) p.units_per_row = cols / 16;
    return p;
}

// ---------------------------------------------------------------------------
struct GemmArgs {
    const void *a_q; int a_fmt, a_lay; int64_t lda;
    const void *b_q; int b_fmt, b_lay; int64_t ldb;
    int64_t M, N, K;
    const float *sa; int sa_gran; const float *sb; int sb_gran;
    const void *bias; int bias_dt;
    void *out; int out_dt; int64_t ldo;
    const float *out_scale; float *out_amax; void *ws;
};

ql_status check_gemm(const GemmArgs &g)
{
    if (!valid_fmt(g.a_fmt) || !valid_fmt(g.b_fmt))
        return fail(QL_ERR_VALUE, "qgemm: unsupported format a=%d b=%d", g.a_fmt, g.b_fmt);
    if ((g.a_fmt == QL_FMT_INT8) != (g.b_fmt == QL_FMT_INT8))
        return fail(QL_ERR_DTYPE, "qgemm: INT8 operands pair only with INT8 (got a=%d b=%d)", g.a_fmt, g.b_fmt);
    if (!valid_layout(g.a_lay) || !valid_layout(g.b_lay))
        return fail(QL_ERR_VALUE, "qgemm: unknown layout a=%d b=%d", g.a_lay, g.b_lay);
    if (!valid_gran(g.sa_gran) || !valid_gran(g.sb_gran))
        return fail(QL_ERR_VALUE, "qgemm: unknown scale granularity sa=%d sb=%d", g.sa_gran, g.sb_gran);
    if (!valid_dtype(g.out_dt)) return fail(QL_ERR_VALUE, "qgemm: unknown output dtype %d", g.out_dt);
    if (g.out_dt == QL_DT_INT32 && g.a_fmt != QL_FMT_INT8)
        return fail(QL_ERR_DTYPE, "qgemm: INT32 output needs INT8 operands");
    if (g.M < 0 || g.N < 0 || g.K < 0)
        return fail(QL_ERR_VALUE, "qgemm: negative size M=%lld N=%lld K=%lld", (long long)g.M, (long long)g.N, (long long)g.K);
    if (g.M > MAX_DIM || g.N > MAX_DIM || g.K > MAX_DIM) return fail(QL_ERR_VALUE, "qgemm: size too large");
    if (g.a_fmt == QL_FMT_INT8 && g.K > INT8_K_MAX)
        return fail(QL_ERR_VALUE, "qgemm: INT8 K=%lld exceeds %lld (INT32 accumulator contract)", (long long)g.K, (long long)INT8_K_MAX);
    const int64_t a_rows = g.a_lay == QL_K_MAJOR ? g.M : g.K, a_cols = g.a_lay == QL_K_MAJOR ? g.K : g.M;
    const int64_t b_rows = g.b_lay == QL_K_MAJOR ? g.N : g.K, b_cols = g.b_lay == QL_K_MAJOR ? g.K : g.N;
    if (a_rows > 0 && g.lda < a_cols)
        return fail(QL_ERR_SHAPE, "qgemm: lda=%lld smaller than the stored row (%lld)", (long long)g.lda, (long long)a_cols);
    if (b_rows > 0 && g.ldb < b_cols)
        return fail(QL_ERR_SHAPE, "qgemm: ldb=%lld smaller than the stored row (%lld)", (long long)g.ldb, (long long)b_cols);
    if (g.M > 0 && g.ldo < g.N)
        return fail(QL_ERR_SHAPE, "qgemm: ldo=%lld smaller than N=%lld", (long long)g.ldo, (long long)g.N);
    if (g.M * g.K > 0 && !g.a_q) return fail(QL_ERR_NULL, "qgemm: a_q is required");
    if (g.N * g.K > 0 && !g.b_q) return fail(QL_ERR_NULL, "qgemm: b_q is required");
    if (g.M * g.N > 0 && !g.out) return fail(QL_ERR_NULL, "qgemm: out is required");
    if (g.out_dt != QL_DT_INT32 && (!g.sa || !g.sb)) return fail(QL_ERR_NULL, "qgemm: sa and sb are required");
    if (g.bias && g.out_dt != QL_DT_INT32 && g.bias_dt != QL_DT_BF16 && g.bias_dt != QL_DT_FP32)
        return fail(QL_ERR_DTYPE, "qgemm: bias must be BF16 or FP32, got dtype %d", g.bias_dt);
    if (g.out_dt == QL_DT_E4M3 && !g.out_scale)
        return fail(QL_ERR_NULL, "qgemm: E4M3 output requires out_scale (the output quantization step)");
    if (g.out_amax && !g.ws) return fail(QL_ERR_NULL, "qgemm: out_amax needs a workspace");
    if ((g.sa_gran == QL_PER_ROW && g.M >= ((int64_t)1 << 32)) || (g.sb_gran == QL_PER_ROW && g.N >= ((int64_t)1 << 32)))
        return fail(QL_ERR_UNSUPPORTED, "qgemm: per-row scales support fewer than 2^32 rows");
    const int64_t bm = 128;
    if (((g.M + bm - 1) / bm) * ((g.N + bm - 1) / bm) > 0x7FFFFFFF)
        return fail(QL_ERR_UNSUPPORTED, "qgemm: output too large for one launch");
    return QL_OK;
}

int out_elem_bytes(int dt) { return dt == QL_DT_BF16 ? 2 : dt == QL_DT_E4M3 ? 1 : 4; }

ql::GemmParams make_gemm(const GemmArgs &g, uint32_t *slot)
{
    ql::GemmParams p{};
    p.a = static_cast<const uint8_t *>(g.a_q);
    p.b = static_cast<const uint8_t *>(g.b_q);
    p.lda = g.lda; p.ldb = g.ldb;
    p.M = g.M; p.N = g.N; p.K = g.K;
    p.sa = g.sa; p.sb = g.sb;
    p.sa_group = g.sa_gran == QL_PER_ROW ? 1 : 0;
    p.sb_group = g.sb_gran == QL_PER_ROW ? 1 : 0;
    p.batch = 1;
    p.bias = g.out_dt == QL_DT_INT32 ? nullptr : g.bias;
    p.bias_dt = p.bias ? g.bias_dt : -1;
    p.out = g.out; p.ldo = g.ldo; p.out_dt = g.out_dt;
    p.out_scale = g.out_scale;
    p.out_amax = g.out_amax;
    p.ws = slot;
    p.amax_part = g.out_amax && g.ws ? ql::ws_amax_parts(g.ws) : nullptr;
    p.a_aligned = aligned16(g.a_q) && g.lda % 16 == 0;
    p.b_aligned = aligned16(g.b_q) && g.ldb % 16 == 0;
    // Fast staging: 16-byte aligned operands whose 16-byte chunks never
    // straddle the matrix edge, and byte offsets that fit the 31-bit buffer
    // range.
    const int64_t lim = (int64_t)1 << 31;
    const bool a_ok = p.a_aligned && (g.a_lay == QL_K_MAJOR ? g.K % 16 == 0 && (g.M + 256) * g.lda < lim
                                                           : g.M % 16 == 0 && (g.K + 256) * g.lda < lim);
    const bool b_ok = p.b_aligned && (g.b_lay == QL_K_MAJOR ? g.K % 16 == 0 && (g.N + 256) * g.ldb < lim
                                                           : g.N % 16 == 0 && (g.K + 256) * g.ldb < lim);
    p.fast = a_ok && b_ok;
    const int eb = out_elem_bytes(g.out_dt);
    p.out_vec4 = (reinterpret_cast<uintptr_t>(g.out) % (uintptr_t)(4 * eb)) == 0 && g.ldo % 4 == 0;
    // 16 consecutive outputs of a row (16-column aligned) are whole 16-byte
    // vectors, and so are 16 consecutive bias entries.
    p.out_vec16 = aligned16(g.out) && (g.ldo * eb) % 16 == 0;
    p.bias_vec16 = p.bias == nullptr || aligned16(p.bias);
    return p;
}

}  // namespace

// ===========================================================================
extern "C" {

size_t ql_workspace_bytes(void) { return (size_t)ql::WS_BYTES; }

ql_status ql_workspace_init(void *ws, size_t bytes, void *stream)
{
    if (!ws) return fail(QL_ERR_NULL, "workspace_init: ws is NULL");
    if (bytes < (size_t)ql::WS_BYTES)
        return fail(QL_ERR_VALUE, "workspace_init: %zu bytes given, %lld needed", bytes, (long long)ql::WS_BYTES);
    return hip_status(ql::launch_ws_zero(ws, ql::WS_COUNTER_BYTES, static_cast<hipStream_t>(stream)),
                      "workspace_init");
}

ql_status ql_quantize(const void *x, ql_dtype x_dt, int64_t rows, int64_t cols, int64_t ldx,
                      ql_gran gran, ql_qfmt fmt, const float *scale_in,
                      void *x_q, int64_t ldq, float *scale_out, float *amax_out,
                      void *ws, void *stream)
{
    ql_status st = check_quantize(x, x_dt, rows, cols, ldx, gran, fmt, scale_in, x_q, ldq, scale_out, ws);
    if (st != QL_OK) return st;
    ql::QzParams p = make_qz(x, x_dt, rows, cols, ldx, gran, fmt, scale_in, x_q, ldq, scale_out, amax_out, ws,
                             ql::WS_SLOT_QA);
    return hip_status(ql::launch_quantize(p, x_dt, fmt, static_cast<hipStream_t>(stream)), "quantize launch");
}

ql_status ql_quantize_ring(const void *x, ql_dtype x_dt, int64_t rows, int64_t cols, int64_t ldx,
                           ql_qfmt fmt, float *ring, int64_t hist_len, int64_t idx, int margin,
                           void *x_q, int64_t ldq, float *scale_used, float *amax_out,
                           void *ws, void *stream)
{
    if (!ring) return fail(QL_ERR_NULL, "quantize_ring: ring is required");
    if (hist_len < 1 || hist_len > RING_MAX_HIST)
        return fail(QL_ERR_VALUE, "quantize_ring: hist_len %lld outside [1, %lld]", (long long)hist_len,
                    (long long)RING_MAX_HIST);
    if (idx < 0 || idx >= hist_len)
        return fail(QL_ERR_VALUE, "quantize_ring: idx %lld outside [0, hist_len)", (long long)idx);
    if (margin < -RING_MAX_MARGIN || margin > RING_MAX_MARGIN)
        return fail(QL_ERR_VALUE, "quantize_ring: margin %d outside [-%d, %d]", margin, RING_MAX_MARGIN,
                    RING_MAX_MARGIN);
    const float *scale_in = ring + hist_len;
    ql_status st = check_quantize(x, x_dt, rows, cols, ldx, QL_PER_TENSOR, fmt, scale_in, x_q, ldq, nullptr, ws);
    if (st != QL_OK) return st;
    ql::QzParams p = make_qz(x, x_dt, rows, cols, ldx, QL_PER_TENSOR, fmt, scale_in, x_q, ldq, nullptr, amax_out,
                             ws, ql::WS_SLOT_QA);
    p.ring = ring;
    p.hist_len = hist_len;
    p.ring_idx = idx;
    p.margin = margin;
    p.scale_used = scale_used;
    return hip_status(ql::launch_quantize(p, x_dt, fmt, static_cast<hipStream_t>(stream)), "quantize_ring launch");
}

ql_status ql_qgemm(const void *a_q, ql_qfmt a_fmt, ql_layout a_lay, int64_t lda,
                   const void *b_q, ql_qfmt b_fmt, ql_layout b_lay, int64_t ldb,
                   int64_t M, int64_t N, int64_t K,
                   const float *sa, ql_gran sa_gran, const float *sb, ql_gran sb_gran,
                   const void *bias, ql_dtype bias_dt,
                   void *out, ql_dtype out_dt, int64_t ldo,
                   const float *out_scale, float *out_amax,
                   void *ws, void *stream)
{
    GemmArgs g{a_q, a_fmt, a_lay, lda, b_q, b_fmt, b_lay, ldb, M, N, K, sa, sa_gran, sb, sb_gran,
               bias, bias_dt, out, out_dt, ldo, out_scale, out_amax, ws};
    ql_status st = check_gemm(g);
    if (st != QL_OK) return st;
    uint32_t *slot = ws ? ql::ws_slot(ws, ql::WS_SLOT_GEMM) : nullptr;
    ql::GemmParams p = make_gemm(g, slot);
    return hip_status(ql::launch_qgemm(p, a_fmt, b_fmt, a_lay == QL_MN_MAJOR, b_lay == QL_MN_MAJOR,
                                       static_cast<hipStream_t>(stream)), "qgemm launch");
}

ql_status ql_linear_forward(const void *x, ql_dtype x_dt, int64_t M, int64_t K,
                            const void *w, int64_t N,
                            const void *bias, ql_dtype bias_dt, ql_qfmt fmt,
                            const float *sx_in, const float *sw_in,
                            void *out, ql_dtype out_dt, const float *out_scale, float *out_amax,
                            void *x_q, float *sx, float *amax_x,
                            void *w_q, float *sw, float *amax_w,
                            void *ws, void *stream)
{
    return (ql_status)ql::linear_forward_ws(x, x_dt, M, K, w, N, bias, bias_dt, fmt, sx_in, sw_in, out, out_dt,
                                            out_scale, out_amax, x_q, sx, amax_x, w_q, sw, amax_w, ws, false,
                                            stream);
}

}  // extern "C"

// Sets the thread's last error (for the entry points in other files).
int ql::report_error(int status, const char *what, const char *detail)
{
    return fail((ql_status)status, "%s: %s", what, detail ? detail : "");
}

// The body of ql_linear_forward.  clear_counters: after validation, first
// zero the workspace's counter slots with a fill kernel (for a workspace
// whose previous contents are not known to be the reset state).
int ql::linear_forward_ws(const void *x, int x_dt, int64_t M, int64_t K, const void *w, int64_t N,
                                const void *bias, int bias_dt, int fmt, const float *sx_in, const float *sw_in,
                                void *out, int out_dt, const float *out_scale, float *out_amax, void *x_q,
                                float *sx, float *amax_x, void *w_q, float *sw, float *amax_w, void *ws,
                                bool clear_counters, void *stream)
{
    if (!ws) return fail(QL_ERR_NULL, "linear_forward: a workspace is required");
    if (!sx || !sw || !amax_x || !amax_w)
        return fail(QL_ERR_NULL, "linear_forward: sx, sw, amax_x and amax_w are required outputs");
    ql_status st = check_quantize(x, x_dt, M, K, K, QL_PER_TENSOR, fmt, sx_in, x_q, K, sx, ws);
    if (st != QL_OK) return st;
    st = check_quantize(w, x_dt, N, K, K, QL_PER_TENSOR, fmt, sw_in, w_q, K, sw, ws);
    if (st != QL_OK) return st;
    GemmArgs g{x_q, fmt, QL_K_MAJOR, K, w_q, fmt, QL_K_MAJOR, K, M, N, K,
               sx_in ? sx_in : sx, QL_PER_TENSOR, sw_in ? sw_in : sw, QL_PER_TENSOR,
               bias, bias_dt, out, out_dt, N, out_scale, out_amax, ws};
    st = check_gemm(g);
    if (st != QL_OK) return st;

    hipStream_t s = static_cast<hipStream_t>(stream);
    if (clear_counters) {
        const hipError_t e = ql::launch_ws_zero(ws, ql::WS_COUNTER_BYTES, s);
        if (e != hipSuccess) return hip_status(e, "linear_forward: clear the workspace counters");
    }
    ql::QzParams px = make_qz(x, x_dt, M, K, K, QL_PER_TENSOR, fmt, sx_in, x_q, K, sx, amax_x,
                              ws, ql::WS_SLOT_QA);
    ql::QzParams pw = make_qz(w, x_dt, N, K, K, QL_PER_TENSOR, fmt, sw_in, w_q, K, sw, amax_w,
                              ws, ql::WS_SLOT_QB);
    // x and w share each pass's launch (one grid row each).
    const hipError_t e = ql::launch_quantize_pair(px, pw, x_dt, fmt, s);
    if (e != hipSuccess) return hip_status(e, "linear_forward: quantize x and w");
    ql::GemmParams pg = make_gemm(g, ql::ws_slot(ws, ql::WS_SLOT_GEMM));
    return hip_status(ql::launch_qgemm(pg, fmt, fmt, 0, 0, s), "linear_forward: qgemm");
}

extern "C" {

ql_status ql_quantize_groups(const void *x, ql_dtype x_dt, int64_t rows, int64_t cols, int64_t ldx,
                             int64_t group_rows, ql_qfmt fmt, const float *scale_in,
                             void *x_q, int64_t ldq, float *scale_out, float *amax_out, void *stream)
{
    if (group_rows < 1) return fail(QL_ERR_VALUE, "quantize_groups: group_rows %lld must be >= 1", (long long)group_rows);
    // Validated as a per-row quantize (no workspace: groups need no election).
    ql_status st = check_quantize(x, x_dt, rows, cols, ldx, QL_PER_ROW, fmt, scale_in, x_q, ldq, scale_out, nullptr);
    if (st != QL_OK) return st;
    if ((rows + group_rows - 1) / group_rows > 0x7FFFFFFF)
        return fail(QL_ERR_UNSUPPORTED, "quantize_groups: at most 2^31-1 groups");
    ql::QzParams p = make_qz(x, x_dt, rows, cols, ldx, QL_PER_ROW, fmt, scale_in, x_q, ldq, scale_out, amax_out,
                             nullptr, 0);
    p.group_rows = group_rows;
    return hip_status(ql::launch_quantize(p, x_dt, fmt, static_cast<hipStream_t>(stream)), "quantize_groups launch");
}

ql_status ql_qgemm_batched(const void *a_q, ql_qfmt a_fmt, ql_layout a_lay, int64_t lda, int64_t stride_a,
                           const void *b_q, ql_qfmt b_fmt, ql_layout b_lay, int64_t ldb, int64_t stride_b,
                           int64_t batch, int64_t M, int64_t N, int64_t K,
                           const float *sa, int64_t group_a, const float *sb, int64_t group_b,
                           const void *bias, ql_dtype bias_dt,
                           void *out, ql_dtype out_dt, int64_t ldo, int64_t stride_out,
                           const float *out_scale, float *out_amax, void *ws, void *stream)
{
    if (batch < 1 || batch > 65535)
        return fail(QL_ERR_VALUE, "qgemm_batched: batch %lld outside [1, 65535]", (long long)batch);
    if (group_a < 0 || group_b < 0)
        return fail(QL_ERR_VALUE, "qgemm_batched: negative scale group size");
    if (stride_a < 0 || stride_b < 0 || stride_out < 0)
        return fail(QL_ERR_VALUE, "qgemm_batched: negative batch stride");
    if (batch * M >= ((int64_t)1 << 32) || batch * N >= ((int64_t)1 << 32))
        return fail(QL_ERR_UNSUPPORTED, "qgemm_batched: batch*M and batch*N must stay below 2^32");
    // Each item is checked as one product; the scale granularity is checked
    // through the group sizes above.
    GemmArgs g{a_q, a_fmt, a_lay, lda, b_q, b_fmt, b_lay, ldb, M, N, K, sa, QL_PER_TENSOR, sb, QL_PER_TENSOR,
               bias, bias_dt, out, out_dt, ldo, out_scale, out_amax, ws};
    ql_status st = check_gemm(g);
    if (st != QL_OK) return st;
    uint32_t *slot = ws ? ql::ws_slot(ws, ql::WS_SLOT_GEMM) : nullptr;
    ql::GemmParams p = make_gemm(g, slot);
    p.sa_group = group_a;
    p.sb_group = group_b;
    p.batch = batch;
    p.stride_a = stride_a;
    p.stride_b = stride_b;
    p.stride_out = stride_out;
    // Every item's base must keep the alignment the vector paths assume.
    if (stride_a % 16) { p.a_aligned = false; p.fast = false; }
    if (stride_b % 16) { p.b_aligned = false; p.fast = false; }
    const int eb = out_elem_bytes(out_dt);
    if (stride_out % 4) p.out_vec4 = false;
    if ((stride_out * eb) % 16) p.out_vec16 = false;
    return hip_status(ql::launch_qgemm(p, a_fmt, b_fmt, a_lay == QL_MN_MAJOR, b_lay == QL_MN_MAJOR,
                                       static_cast<hipStream_t>(stream)), "qgemm_batched launch");
}

ql_status ql_linear_forward_static(const void *x, ql_dtype x_dt, int64_t M, int64_t K,
                                  const void *w_q, int64_t N, const float *sw,
                                  const void *bias, ql_dtype bias_dt, const float *bias_scale,
                                  ql_qfmt fmt, const float *sx_in,
                                  void *out, ql_dtype out_dt, const float *out_scale, float *out_amax,
                                  void *x_q, float *sx, float *amax_x, void *ws, void *stream)
{
    if (!valid_fmt(fmt)) return fail(QL_ERR_VALUE, "linear_forward_static: unsupported format %d", fmt);
    if (fmt == QL_FMT_INT8) return fail(QL_ERR_DTYPE, "linear_forward_static: FP8 formats only");
    if (!ws) return fail(QL_ERR_NULL, "linear_forward_static: a workspace is required");
    if (!sx || !amax_x) return fail(QL_ERR_NULL, "linear_forward_static: sx and amax_x are required outputs");
    if (!sw) return fail(QL_ERR_NULL, "linear_forward_static: sw (the weight's step) is required");
    ql_status st = check_quantize(x, x_dt, M, K, K, QL_PER_TENSOR, fmt, sx_in, x_q, K, sx, ws);
    if (st != QL_OK) return st;
    const bool qbias = bias && bias_scale;
    // A quantized bias is checked as "no bias" here and attached below.
    GemmArgs g{x_q, fmt, QL_K_MAJOR, K, w_q, fmt, QL_K_MAJOR, K, M, N, K,
               sx_in ? sx_in : sx, QL_PER_TENSOR, sw, QL_PER_TENSOR,
               qbias ? nullptr : bias, bias_dt, out, out_dt, N, out_scale, out_amax, ws};
    st = check_gemm(g);
    if (st != QL_OK) return st;

    hipStream_t s = static_cast<hipStream_t>(stream);
    ql::QzParams px = make_qz(x, x_dt, M, K, K, QL_PER_TENSOR, fmt, sx_in, x_q, K, sx, amax_x,
                              ws, ql::WS_SLOT_QA);
    hipError_t e = ql::launch_quantize(px, x_dt, fmt, s);
    if (e != hipSuccess) return hip_status(e, "linear_forward_static: quantize x");
    ql::GemmParams pg = make_gemm(g, ql::ws_slot(ws, ql::WS_SLOT_GEMM));
    if (qbias && out_dt != QL_DT_INT32) {
        pg.bias = bias;
        pg.bias_dt = fmt == QL_FMT_E4M3 ? ql::BIAS_Q_E4M3 : ql::BIAS_Q_E5M2;
        pg.bias_scale = bias_scale;
        pg.bias_vec16 = aligned16(bias);
    }
    return hip_status(ql::launch_qgemm(pg, fmt, fmt, 0, 0, s), "linear_forward_static: qgemm");
}

ql_status ql_linear_backward(const void *g, int64_t M, int64_t N,
                             const void *x_q, ql_qfmt x_fmt, const float *sx,
                             const void *w_q, ql_qfmt w_fmt, const float *sw, int64_t K,
                             unsigned masks, ql_qfmt g_fmt, const float *sg_in,
                             void *dx, void *dw, ql_dtype out_dt, float *dbias,
                             void *g_q, float *sg, float *amax_g, void *ws, void *stream)
{
    if (masks == 0 || (masks & ~7u))
        return fail(QL_ERR_VALUE, "linear_backward: masks %u must be a non-empty subset of 1|2|4", masks);
    const bool want_dx = masks & QL_BWD_DX, want_dw = masks & QL_BWD_DW, want_db = masks & QL_BWD_DBIAS;
    if (out_dt != QL_DT_BF16 && out_dt != QL_DT_FP32)
        return fail(valid_dtype(out_dt) ? QL_ERR_DTYPE : QL_ERR_VALUE,
                    "linear_backward: gradients are BF16 or FP32, got dtype %d", out_dt);
    if (g_fmt == QL_FMT_INT8 || x_fmt == QL_FMT_INT8 || w_fmt == QL_FMT_INT8)
        return fail(valid_fmt(g_fmt) && valid_fmt(x_fmt) && valid_fmt(w_fmt) ? QL_ERR_DTYPE : QL_ERR_VALUE,
                    "linear_backward: FP8 formats only");
    if (K < 0) return fail(QL_ERR_VALUE, "linear_backward: negative K");
    ql_status st;
    if (want_db) {
        if (M < 0 || N < 0) return fail(QL_ERR_VALUE, "linear_backward: negative size");
        if (!dbias && N > 0) return fail(QL_ERR_NULL, "linear_backward: dbias is required by the mask");
        if (!g && M > 0 && N > 0) return fail(QL_ERR_NULL, "linear_backward: g is required");
        if (!ws && N > 0) return fail(QL_ERR_NULL, "linear_backward: grad_bias needs a workspace");
    }
    const bool gemms = want_dx || want_dw;
    GemmArgs gx{}, gw{};
    if (gemms) {
        if (!sg || !amax_g) return fail(QL_ERR_NULL, "linear_backward: sg and amax_g are required outputs");
        st = check_quantize(g, QL_DT_BF16, M, N, N, QL_PER_TENSOR, g_fmt, sg_in, g_q, N, sg, ws);
        if (st != QL_OK) return st;
        const float *sg_use = sg_in ? sg_in : sg;
        // dX [M, K] = g [M, N] . W: A = g codes (K-major over n), B[k, n] =
        // W[n, k] read MN-major from w_q [N, K].
        gx = GemmArgs{g_q, g_fmt, QL_K_MAJOR, N, w_q, w_fmt, QL_MN_MAJOR, K, M, K, N,
                      sg_use, QL_PER_TENSOR, sw, QL_PER_TENSOR, nullptr, QL_DT_FP32, dx, out_dt, K,
                      nullptr, nullptr, ws};
        // dW [N, K] = g^T . X: A[n, m] = g[m, n] read MN-major from the g
        // codes, B[k, m] = X[m, k] read MN-major from x_q [M, K].
        gw = GemmArgs{g_q, g_fmt, QL_MN_MAJOR, N, x_q, x_fmt, QL_MN_MAJOR, K, N, K, M,
                      sg_use, QL_PER_TENSOR, sx, QL_PER_TENSOR, nullptr, QL_DT_FP32, dw, out_dt, K,
                      nullptr, nullptr, ws};
        if (want_dx && (st = check_gemm(gx)) != QL_OK) return st;
        if (want_dw && (st = check_gemm(gw)) != QL_OK) return st;
    }

    hipStream_t s = static_cast<hipStream_t>(stream);
    if (gemms) {
        ql::QzParams pg = make_qz(g, QL_DT_BF16, M, N, N, QL_PER_TENSOR, g_fmt, sg_in, g_q, N, sg, amax_g,
                                  ws, ql::WS_SLOT_QA);
        hipError_t e = ql::launch_quantize(pg, QL_DT_BF16, g_fmt, s);
        if (e != hipSuccess) return hip_status(e, "linear_backward: quantize g");
        if (want_dx) {
            ql::GemmParams p = make_gemm(gx, nullptr);
            e = ql::launch_qgemm(p, g_fmt, w_fmt, 0, 1, s);
            if (e != hipSuccess) return hip_status(e, "linear_backward: dX");
        }
        if (want_dw) {
            ql::GemmParams p = make_gemm(gw, nullptr);
            e = ql::launch_qgemm(p, g_fmt, x_fmt, 1, 1, s);
            if (e != hipSuccess) return hip_status(e, "linear_backward: dW");
        }
    }
    if (want_db && M >= 0 && N > 0) {
        hipError_t e = ql::launch_col_sum_bf16(g, M, N, N, dbias, ql::ws_partials(ws), s);
        if (e != hipSuccess) return hip_status(e, "linear_backward: grad_bias");
    }
    return QL_OK;
}

const char *ql_status_string(ql_status s)
{
    switch (s) {
    case QL_OK: return "ok";
    case QL_ERR_VALUE: return "invalid value";
    case QL_ERR_DTYPE: return "unsupported dtype or format combination";
    case QL_ERR_SHAPE: return "invalid shape or leading dimension";
    case QL_ERR_NULL: return "required pointer is NULL";
    case QL_ERR_UNSUPPORTED: return "unsupported";
    case QL_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char *ql_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
