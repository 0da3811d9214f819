// internal.hpp -- parameter blocks and launchers shared between the C-ABI
// front end (qlinear_api.cpp) and the kernel files.  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ql {

// Quantized bias (static inference): codes of the layer's format times a
// per-tensor step.
enum : int { BIAS_Q_E4M3 = 16, BIAS_Q_E5M2 = 17 };

// Workspace layout: slots of 256 bytes, each {amax bits, counter, ...}.
constexpr int64_t WS_SLOT_BYTES = 256;
constexpr int64_t WS_SLOT_QA = 0;      // quantize of x / A
constexpr int64_t WS_SLOT_QB = 1;      // quantize of w / B (linear_forward)
constexpr int64_t WS_SLOT_GEMM = 2;    // GEMM output amax
constexpr int64_t WS_COUNTER_BYTES = 4 * WS_SLOT_BYTES;   // zeroed once, left zeroed by every call
// Partial column sums of grad_bias (no zeroing needed: fully overwritten).
constexpr int64_t WS_PART_BYTES = (int64_t)1 << 20;
// Per-workgroup maxima of a GEMM's out_amax (fully overwritten per call).
constexpr int64_t WS_AMAX_PARTS = (int64_t)1 << 16;
constexpr int64_t WS_BYTES = WS_COUNTER_BYTES + WS_PART_BYTES + WS_AMAX_PARTS * 4;

inline float *ws_partials(void *ws) { return reinterpret_cast<float *>(static_cast<char *>(ws) + WS_COUNTER_BYTES); }
// Per-tensor quantize: its workgroups' maxima at ws_amax_parts + slot *
// QZ_PARTS_PER_SLOT (at most QZ_MAX_BLOCKS of them).
constexpr int64_t QZ_PARTS_PER_SLOT = 1024;
inline uint32_t *ws_amax_parts(void *ws)
{
    return reinterpret_cast<uint32_t *>(static_cast<char *>(ws) + WS_COUNTER_BYTES + WS_PART_BYTES);
}

inline uint32_t *ws_slot(void *ws, int64_t slot)
{
    return reinterpret_cast<uint32_t *>(static_cast<char *>(ws) + slot * WS_SLOT_BYTES);
}

struct QzParams {
    const void *x;
    int64_t rows, cols, ldx;
    void *xq;
    int64_t ldq;
    const float *scale_src;   // step the cast uses: scale_out (current) or scale_in (delayed)
    float *scale_out;         // fl32(amax / qmax)
    float *amax_out;
    uint32_t *ws;             // workspace slot (per-tensor only)
    float qmax, floor;
    int64_t n_elems;          // rows * cols
    int64_t n_units;          // 16-element vector units (flat / rows modes)
    int64_t units_per_row;    // cols / 16 (rows mode, per-row vector path)
    int mode;                 // 0 flat-vector, 1 rows-vector, 2 scalar
    int per_row;              // one scale per group of group_rows rows (per row: 1)
    int64_t group_rows;
    int vec_rows;             // per-row kernel may use 16-byte units
    int delayed;
    // Delayed scaling with an amax history ring [hist (hist_len) | scale]:
    // the cast reads the scale from ring[hist_len] (scale_src), and the last
    // workgroup stores amax at hist[ring_idx], writes the scale it used to
    // scale_used and publishes fl32(max(hist)/qmax) * 2^margin.
    float *ring;
    int64_t hist_len, ring_idx;
    int margin;
    float *scale_used;
    // Current scaling on large grids: workgroup w of the amax pass stores
    // its maximum at amax_part[w] and every workgroup of the cast pass
    // reduces them (null: the last-workgroup election).
    uint32_t *amax_part;
};

// Up to two whole-tensor quantizes in one launch per pass (grid row y
// works on tensor y, each with its own workspace slot and election).
struct QzPack {
    QzParams t[2];
};

hipError_t launch_quantize(const QzParams &p, int in_dt, int fmt, hipStream_t s);
// Quantize two tensors of the same input dtype and format: one launch per
// pass when both are whole-tensor quantizes of the same kind, else one
// after the other.
hipError_t launch_quantize_pair(const QzParams &p0, const QzParams &p1, int in_dt, int fmt, hipStream_t s);
// grad_bias: out[n] = sum_m g[m, n] for BF16 g [M, N] (leading dimension ldg);
// partials: WS_PART_BYTES of scratch (the workspace's partial area).
hipError_t launch_col_sum_bf16(const void *g, int64_t M, int64_t N, int64_t ldg, float *out, float *partials,
                               hipStream_t s);
hipError_t launch_ws_zero(void *ws, int64_t bytes, hipStream_t s);

// Unsigned division by a divisor d fixed for a launch, as a multiply-high
// and a shift (Granlund and Montgomery, "Division by invariant integers
// using multiplication", PLDI 1994, section 4): with l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1, n / d = (mulhi(n, m) + n) >> l for every
// n < 2^32 (the sum is formed in 64 bits, so it cannot overflow).  d = 0
// stands for "one scale": the quotient is 0.
struct GroupDiv {
    uint32_t d, m;
    int l;
    __host__ __device__ void init(int64_t div)
    {
        d = (uint32_t)div;
        l = 0;
        while (l < 32 && ((uint64_t)1 << l) < (uint64_t)d) ++l;
        m = d ? (uint32_t)((((uint64_t)1 << 32) * (((uint64_t)1 << l) - d)) / d + 1) : 0;
    }
    __host__ __device__ uint32_t operator()(uint32_t n) const
    {
        if (d == 0) return 0;
        const uint64_t t = ((uint64_t)n * m) >> 32;
        return (uint32_t)((t + n) >> l);
    }
};

struct GemmParams {
    const uint8_t *a, *b;
    int64_t lda, ldb;
    int64_t M, N, K;
    const float *sa, *sb;
    int64_t sa_group, sb_group;     // rows per scale: 0 (one scale), 1 (per row), G (row groups)
    GroupDiv sa_div, sb_div;        // the same divisions (launch_qgemm fills them)
    // Batched products (grid y = batch index z): item z reads a + z*stride_a,
    // b + z*stride_b and writes out + z*stride_out (elements); its scale
    // rows are z*M + m and z*N + n of the flattened batch.
    int64_t batch;                  // batch items (grid y); 1 for a single product
    int64_t stride_a, stride_b, stride_out;
    int64_t row_base, col_base;     // z*M, z*N (set in the kernel)
    const void *bias;
    int bias_dt;                    // -1 none, 0 BF16, 1 FP32, BIAS_Q_E4M3 / BIAS_Q_E5M2 codes
    const float *bias_scale;        // step of a quantized bias ([1])
    void *out;
    int64_t ldo;
    int out_dt;                     // DT_BF16 / DT_FP32 / DT_E4M3 / DT_INT32
    const float *out_scale;
    float *out_amax;
    uint32_t *ws;                   // workspace slot for the out_amax election
    // out_amax without an election: workgroup w stores its maximum at
    // amax_part[w] and a one-workgroup kernel reduces them after the GEMM
    // (null: the last-workgroup election; see gemm_amax_parts).
    uint32_t *amax_part;
    int a_aligned, b_aligned;       // 16-byte loads allowed
    int out_vec4;                   // 4 consecutive outputs may be stored as one vector
    int out_vec16;                  // 16 consecutive outputs (16-aligned column) are 16-byte vectors
    int bias_vec16;                 // bias absent or 16-byte aligned
    int fast;                       // branch-free buffer-load staging applies
    int tiles_m, tiles_n;
};

// Fills sa_div / sb_div from sa_group / sb_group; scale rows (z*M + m and
// z*N + n) must stay below 2^32.
inline void finish_groups(GemmParams &p)
{
    p.sa_div.init(p.sa_group);
    p.sb_div.init(p.sb_group);
}

// out_amax of a GEMM whose nblocks workgroups stored their maxima at
// p.amax_part (run right after the GEMM on the same stream).
hipError_t launch_amax_finalize(const GemmParams &p, int64_t nblocks, hipStream_t s);

// Grids of at most this many workgroups (one wave of them on 256 CUs at two
// per CU) publish out_amax by the last-workgroup election; the election's
// atomics are serialized at the memory side, and in a grid that runs in
// several waves each wave's workgroups would hold their CUs while they
// queue.  Larger grids (and grids larger than the workspace array) keep
// per-workgroup maxima and the finalize launch.
constexpr int64_t GEMM_ELECT_MAX_BLOCKS = 512;
inline uint32_t *gemm_amax_parts(uint32_t *parts, int64_t blocks)
{
    return blocks <= GEMM_ELECT_MAX_BLOCKS || blocks > WS_AMAX_PARTS ? nullptr : parts;
}

// Compute units of the current device (cached per device; 256 if the query
// fails), the size of a persistent grid of one workgroup per CU.
int device_cu_count();

// The body of ql_linear_forward (enum arguments as int; the status as int,
// a ql_status value).  clear_counters: zero the workspace's counter slots
// (a fill kernel) after validation and before the work.
int linear_forward_ws(const void *x, int x_dt, int64_t M, int64_t K, const void *w, int64_t N, const void *bias,
                      int bias_dt, int fmt, const float *sx_in, const float *sw_in, void *out, int out_dt,
                      const float *out_scale, float *out_amax, void *x_q, float *sx, float *amax_x, void *w_q,
                      float *sw, float *amax_w, void *ws, bool clear_counters, void *stream);

// Records "what: detail" as the calling thread's last error and returns
// status (a ql_status value).
int report_error(int status, const char *what, const char *detail);

// a_fmt / b_fmt: FMT_*; a_mn / b_mn: operand stored MN-major.
hipError_t launch_qgemm(const GemmParams &p, int a_fmt, int b_fmt, int a_mn, int b_mn, hipStream_t s);

}  // namespace ql
