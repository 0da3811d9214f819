// qgemm_impl.hpp -- the general scaled FP8 / INT8 matrix-core GEMM kernel
// for gfx950 (every layout and alignment), and the per-shape dispatch.
//
//   out[m, n] = (sum_k A[m, k] * B[n, k]) * sa[m|0] * sb[n|0] (+ bias[n])
//
// AstrAI ops/fp8.py @5e76fbd: fp8_gemm / mm_fp8 (a @ b * (sa*sb), FP32
// accumulation, BF16 or E4M3 output where E4M3 divides by out_scale, the
// output quantization step) and linear_forward_fp8 (bias fused into the GEMM
// epilogue); scmp_kernels README "API" (a @ b.T, per-row scales).
//
// Design (one workgroup = 4 waves = one BM x BN output tile):
//   * K advances in steps of 128 bytes.  Each step's A and B tiles are
//     staged in LDS, double buffered, from two register sets: the global
//     loads of step k+2 are in flight while the matrix cores work on step k.
//   * LDS holds every operand K-major (128 bytes per row) with a 16-byte
//     chunk swizzle, so the fragment reads (one row per lane, two 16-byte
//     chunks) are free of bank conflicts.  MN-major operands reach this
//     kernel only when unaligned or ragged (aligned ones take the
//     direct-to-LDS kernel); they are bounds-checked and transposed in
//     registers (byte permutes) on their way into LDS.
//   * FP8: v_mfma_f32_16x16x128_f8f6f4 with per-operand formats (E4M3 and
//     E5M2 mix freely).  INT8: two v_mfma_i32_16x16x64_i8 per 128 bytes,
//     exact in INT32.  Each lane's 32 fragment bytes are 32 consecutive k, so
//     the matrix core's groups of 8 products are 8 consecutive k.
//   * Tile order: tiles are grouped GM tile-rows at a time so a run of
//     workgroups shares A rows and B columns, and consecutive tiles of that
//     order are placed on the same XCD (workgroup ids go round-robin over
//     the 8 XCDs, each with its own L2).  This is the gfx950 form of the
//     grouped rasterization the AstrAI commit message describes.
//   * Epilogue: scale, bias and the output cast fused; optional max|v| of
//     the output published by the last workgroup (same election as the
//     quantize reduction).
#pragma once

#include "qgemm_common.hpp"

#include <type_traits>

namespace ql {

constexpr int GEMM_BK = 128;
__device__ __forceinline__ int lds_swz(int r) { return (r & 7) ^ ((r >> 3) & 7); }
__device__ __forceinline__ int lds_off(int r, int chunk) { return r * GEMM_BK + ((chunk ^ lds_swz(r)) << 4); }

// MN-major operand in LDS (direct-to-LDS kernel): stored as it lies in
// memory, one row of R mn-bytes per k, with its 16-byte chunks XOR-swizzled
// by a function of k so that its transpose reads (8 k-rows at one mn offset
// per 16-lane block, two blocks served together) hit distinct banks;
// brute-force checked for 16- and 32-lane groups.
template <int R> __device__ __forceinline__ int mn_swz(int kr)
{
    static_assert(R == 256 || R == 128 || R == 64, "MN-major tile rows");
    if constexpr (R == 256) return (kr & 7) | (((kr >> 5) & 1) << 3);
    else if constexpr (R == 128) return ((kr >> 1) & 3) | (((kr >> 5) & 1) << 2);
    else return ((kr >> 2) & 1) | (((kr >> 5) & 1) << 1);
}

// Load up to 16 bytes [p, p + n) into a zero-padded 16-byte vector.
__device__ __forceinline__ uint4 load_partial(const uint8_t *p, int64_t n)
{
    uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 16; ++i)
        if (i < n) w[i >> 2] |= (uint32_t)p[i] << (8 * (i & 3));
    return make_uint4(w[0], w[1], w[2], w[3]);
}

__device__ __forceinline__ uint32_t word_of(const uint4 &v, int i)
{
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Byte transpose of a 4 x 4 block: row j is word r[j] (byte b = column b);
// c[b] collects column b, row j in byte j.  Two rounds of v_perm_b32, whose
// selector byte i picks byte i of the result from the 8 bytes {hi : lo}
// (0..3 = lo's bytes, 4..7 = hi's).
__device__ __forceinline__ void transpose_4x4_bytes(uint32_t r0, uint32_t r1, uint32_t r2, uint32_t r3,
                                                    uint32_t (&c)[4])
{
    const uint32_t t0 = __builtin_amdgcn_perm(r1, r0, 0x06020400u);   // r0.0 r1.0 r0.2 r1.2
    const uint32_t t1 = __builtin_amdgcn_perm(r1, r0, 0x07030501u);   // r0.1 r1.1 r0.3 r1.3
    const uint32_t t2 = __builtin_amdgcn_perm(r3, r2, 0x06020400u);   // r2.0 r3.0 r2.2 r3.2
    const uint32_t t3 = __builtin_amdgcn_perm(r3, r2, 0x07030501u);   // r2.1 r3.1 r2.3 r3.3
    c[0] = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
    c[1] = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
    c[2] = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
    c[3] = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
}

// 8 k-rows x 16 mn-bytes (r[j] = k-row j) -> 16 mn-rows of 8 k-bytes:
// lo[e] holds k-rows 0..3 of mn-row e, hi[e] k-rows 4..7.
__device__ __forceinline__ void transpose_8x16_bytes(const uint4 (&r)[8], uint32_t (&lo)[16], uint32_t (&hi)[16])
{
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        uint32_t c[4];
        transpose_4x4_bytes(word_of(r[0], w), word_of(r[1], w), word_of(r[2], w), word_of(r[3], w), c);
#pragma unroll
        for (int b = 0; b < 4; ++b) lo[4 * w + b] = c[b];
        transpose_4x4_bytes(word_of(r[4], w), word_of(r[5], w), word_of(r[6], w), word_of(r[7], w), c);
#pragma unroll
        for (int b = 0; b < 4; ++b) hi[4 * w + b] = c[b];
    }
}

// ---------------------------------------------------------------------------
// Stage one K step of one operand ([ROWS, 128 bytes] of the logical [MN, K]
// matrix) from global memory into registers, then into LDS.
template <int ROWS, bool MN_MAJOR> struct Stage;

// K-major: 8 threads read one row's 128 contiguous bytes.
template <int ROWS> struct Stage<ROWS, false> {
    static constexpr int PER = ROWS * 8 / GEMM_THREADS;
    uint4 r[PER];
    __device__ __forceinline__ void load(const uint8_t *base, int64_t ld, int64_t row0, int64_t rows_total,
                                         int64_t k0, int64_t K, bool aligned)
    {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int c = i * GEMM_THREADS + (int)threadIdx.x;
            const int64_t grow = row0 + (c >> 3);
            const int64_t gk = k0 + (c & 7) * 16;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (grow < rows_total && gk < K) {
                const uint8_t *src = base + grow * ld + gk;
                if (aligned && gk + 16 <= K) v = *reinterpret_cast<const uint4 *>(src);
                else v = load_partial(src, K - gk);
            }
            r[i] = v;
        }
    }
    __device__ __forceinline__ void store(uint8_t *lds) const
    {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int c = i * GEMM_THREADS + (int)threadIdx.x;
            *reinterpret_cast<uint4 *>(lds + lds_off(c >> 3, c & 7)) = r[i];
        }
    }
};

// MN-major (storage [K][MN]): a thread reads 8 k-rows x 16 mn-bytes and
// transposes them to 16 rows of 8 consecutive k.
template <int ROWS> struct Stage<ROWS, true> {
    static constexpr int GROUPS = ROWS / 16;                     // 16-byte mn groups
    static constexpr int UNITS = GROUPS * (GEMM_BK / 8);         // = ROWS
    static constexpr int PER = (UNITS + GEMM_THREADS - 1) / GEMM_THREADS;
    uint4 r[PER][8];
    __device__ __forceinline__ void load(const uint8_t *base, int64_t ld, int64_t row0, int64_t rows_total,
                                         int64_t k0, int64_t K, bool aligned)
    {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int u = i * GEMM_THREADS + (int)threadIdx.x;
            const int mg = u % GROUPS, kq = u / GROUPS;
            const int64_t mn = row0 + mg * 16;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int64_t k = k0 + kq * 8 + j;
                uint4 v = make_uint4(0, 0, 0, 0);
                if (u < UNITS && k < K && mn < rows_total) {
                    const uint8_t *src = base + k * ld + mn;
                    if (aligned && mn + 16 <= rows_total) v = *reinterpret_cast<const uint4 *>(src);
                    else v = load_partial(src, rows_total - mn);
                }
                r[i][j] = v;
            }
        }
    }
    __device__ __forceinline__ void store(uint8_t *lds) const
    {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int u = i * GEMM_THREADS + (int)threadIdx.x;
            if (u >= UNITS) continue;
            const int mg = u % GROUPS, kq = u / GROUPS;
            uint32_t lo[16], hi[16];
            transpose_8x16_bytes(r[i], lo, hi);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = mg * 16 + e;
                *reinterpret_cast<uint2 *>(lds + lds_off(row, kq >> 1) + (kq & 1) * 8) = make_uint2(lo[e], hi[e]);
            }
        }
    }
};

// ---------------------------------------------------------------------------
// Branch-free staging through buffer loads (the fast path).
//
// A buffer resource covers the operand from the tile's first row (or
// column) on, with num_records set so that rows past the matrix fall outside
// it; the hardware returns zeros for out-of-range loads, so no bounds test
// is needed per load.  Chunks past K (the last K step) get an offset far
// outside the range.  Needs 16-byte aligned operands, leading dimensions and
// K (K-major) or MN extent (MN-major) that are multiples of 16, and byte
// offsets below 2^31 (checked on the host).  BUF_OOB / BUF_WORD3 are in
// qgemm_common.hpp.
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}

template <int ROWS, bool MN_MAJOR> struct FastStage;

template <int ROWS> struct FastStage<ROWS, false> {
    static constexpr int PER = ROWS * 8 / GEMM_THREADS;
    uint4 r[PER];
    __amdgpu_buffer_rsrc_t rsrc;
    uint32_t off[PER];      // row * ld + chunk * 16, tile relative
    int kc;                 // this thread's chunk start within a K step
    __device__ __forceinline__ void init(const uint8_t *base, int64_t ld, int64_t row0, int64_t rows_total, int64_t K)
    {
        const int64_t rows_left = rows_total - row0;
        const int64_t bytes = rows_left > 0 ? rows_left * ld : 0;
        rsrc = __builtin_amdgcn_make_buffer_rsrc((void *)(base + row0 * ld), (short)0,
                                                 (int)(bytes < 0x7FFFFFFF ? bytes : 0x7FFFFFFF), BUF_WORD3);
        kc = ((int)threadIdx.x & 7) * 16;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int c = i * GEMM_THREADS + (int)threadIdx.x;
            off[i] = (uint32_t)((c >> 3) * ld + kc);
        }
        (void)K;
    }
    __device__ __forceinline__ void load(int64_t k0, int64_t K)
    {
        const bool in_k = k0 + kc < K;
#pragma unroll
        for (int i = 0; i < PER; ++i) r[i] = buf_load16(rsrc, in_k ? off[i] + (uint32_t)k0 : BUF_OOB);
    }
    __device__ __forceinline__ void store(uint8_t *lds) const
    {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int c = i * GEMM_THREADS + (int)threadIdx.x;
            *reinterpret_cast<uint4 *>(lds + lds_off(c >> 3, c & 7)) = r[i];
        }
    }
};

// Generic staging adapter with the same interface (odd shapes, unaligned
// operands): bounds-checked loads with a byte-wise fallback.
template <int ROWS, bool MN_MAJOR> struct SafeStage {
    Stage<ROWS, MN_MAJOR> st;
    const uint8_t *base;
    int64_t ld, row0, rows_total;
    bool aligned;
    __device__ __forceinline__ void init(const uint8_t *b, int64_t l, int64_t r0, int64_t rt, int64_t K)
    {
        base = b; ld = l; row0 = r0; rows_total = rt;
        (void)K;
    }
    __device__ __forceinline__ void load(int64_t k0, int64_t K) { st.load(base, ld, row0, rows_total, k0, K, aligned); }
    __device__ __forceinline__ void store(uint8_t *lds) const { st.store(lds); }
};

// ---------------------------------------------------------------------------
template <int AF, int BF> struct Mma {
    typedef v4f acc_t;
    __device__ __forceinline__ static void run(acc_t &c, const v8i &a, const v8i &b)
    {
        c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, AF, BF, 0, 0, 0, 0);
    }
    static constexpr bool INT_ACC = false;
    __device__ __forceinline__ static uint32_t bits(const acc_t &c, int r) { return __float_as_uint(c[r]); }
};

template <> struct Mma<FMT_INT8, FMT_INT8> {
    typedef v4i acc_t;
    __device__ __forceinline__ static void run(acc_t &c, const v8i &a, const v8i &b)
    {
        v4i a0 = {a[0], a[1], a[2], a[3]}, a1 = {a[4], a[5], a[6], a[7]};
        v4i b0 = {b[0], b[1], b[2], b[3]}, b1 = {b[4], b[5], b[6], b[7]};
        c = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b0, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b1, c, 0, 0, 0);
    }
    static constexpr bool INT_ACC = true;
    __device__ __forceinline__ static uint32_t bits(const acc_t &c, int r) { return (uint32_t)c[r]; }
};

// Fragment of 16 rows x 32 k for lane l: row (l & 15), k = 32*(l >> 4) .. +31.
__device__ __forceinline__ v8i load_frag(const uint8_t *lds, int row, int g)
{
    uint4 x = *reinterpret_cast<const uint4 *>(lds + lds_off(row, 2 * g));
    uint4 y = *reinterpret_cast<const uint4 *>(lds + lds_off(row, 2 * g + 1));
    v8i f = {(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
    return f;
}

// Batch item z (grid y): its operands, its output and its scale rows.
__device__ __forceinline__ void select_batch_item(GemmParams &p)
{
    const int64_t z = blockIdx.y;
    const int eb = p.out_dt == DT_BF16 ? 2 : p.out_dt == DT_E4M3 ? 1 : 4;
    p.a += z * p.stride_a;
    p.b += z * p.stride_b;
    p.out = static_cast<char *>(p.out) + z * p.stride_out * eb;
    p.row_base = z * p.M;
    p.col_base = z * p.N;
}

// Epilogue of a wave's TM x TN grid of 16 x 16 accumulators (16x16x128
// layout: element r of lane (lr, g) is row 4g + r, column lr), one 16-row
// slab at a time: the slab goes to a per-wave LDS area (raw FP32 / INT32
// bits), then each lane takes 4 consecutive columns of a row, so stores are
// contiguous along rows.  Reuses `lds` (every wave must be done with it),
// and ends with the optional out_amax election.
template <typename MMA, int TM, int TN, int WN>
__device__ __forceinline__ void epilogue_tile(const GemmParams &p, uint8_t *lds, uint32_t *red,
                                              typename MMA::acc_t (&acc)[TM][TN], int64_t row0, int64_t col0,
                                              int wave, int lane)
{
    const int lr = lane & 15, g = lane >> 4;
    constexpr int EP_LD = WN + 4;                       // padded row, in words
    uint32_t *ep = reinterpret_cast<uint32_t *>(lds) + wave * 16 * EP_LD;
    Epilogue epi(p);
    uint32_t vmax = 0;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        __syncthreads();
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                ep[(g * 4 + r) * EP_LD + j * 16 + lr] = MMA::bits(acc[i][j], r);
        __syncthreads();
        constexpr int C4 = WN / 4;                       // 4-column groups per row
#pragma unroll 1
        for (int idx = lane; idx < 16 * C4; idx += 64) {
            const int rr = idx / C4, c4 = idx - rr * C4;
            const uint4 w = *reinterpret_cast<const uint4 *>(ep + rr * EP_LD + c4 * 4);
            const int64_t row = row0 + i * 16 + rr;
            const int64_t col = col0 + c4 * 4;
            if (row < p.M && col < p.N) vmax = epi.store4<MMA::INT_ACC>(w, row, col, vmax);
        }
    }
    if (p.out_amax) gemm_publish_amax(p, vmax, red);
}

template <int AF, int BF, bool A_MN, bool B_MN, int BM, int BN, int MINW, bool FAST, int PF>
__global__ __launch_bounds__(GEMM_THREADS, MINW) void qgemm_kernel(GemmParams p)
{
    typedef Mma<AF, BF> MMA;
    typedef typename MMA::acc_t acc_t;
    constexpr int WM = BM / 2, WN = BN / 2, TM = WM / 16, TN = WN / 16;
    constexpr int STAGE = (BM + BN) * GEMM_BK;
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE];
    __shared__ uint32_t red[GEMM_THREADS / 64];

    select_batch_item(p);
    int tm, tn;
    tile_coords(p.tiles_m, p.tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm0 = (wave >> 1) * WM, wn0 = (wave & 1) * WN;
    const int lr = lane & 15, g = lane >> 4;

    acc_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = acc_t{0, 0, 0, 0};

    typedef typename std::conditional<FAST, FastStage<BM, A_MN>, SafeStage<BM, A_MN> >::type StageA;
    typedef typename std::conditional<FAST, FastStage<BN, B_MN>, SafeStage<BN, B_MN> >::type StageB;
    // PF = 2: two register sets per operand, so the global loads of step
    // k+2 are issued while step k is computed and step k+1 goes from
    // registers to LDS (each load has two steps to arrive).  PF = 1: one set,
    // step k+1's loads overlap step k.  Loads past K read zeros (bounds
    // checks, or offsets outside the buffer range).
    static_assert(PF == 1 || PF == 2, "prefetch depth");
    StageA sa0, sa1;
    StageB sb0, sb1;
    sa0.init(p.a, p.lda, m0, p.M, p.K);
    sb0.init(p.b, p.ldb, n0, p.N, p.K);
    if constexpr (!FAST) { sa0.aligned = p.a_aligned; sb0.aligned = p.b_aligned; }
    if constexpr (PF == 2) { sa1 = sa0; sb1 = sb0; }
    const int nk = (int)((p.K + GEMM_BK - 1) / GEMM_BK);
    if (nk > 0) {
        sa0.load(0, p.K);
        sb0.load(0, p.K);
        if constexpr (PF == 2) {
            sa1.load(GEMM_BK, p.K);
            sb1.load(GEMM_BK, p.K);
        }
        sa0.store(lds);
        sb0.store(lds + BM * GEMM_BK);
    }
    __syncthreads();
    // Step kt: reload set r with step kt + PF, compute step kt from LDS,
    // store set n (step kt + 1) into the other LDS buffer.
    auto step = [&](int kt, StageA &ra, StageB &rb, StageA &na, StageB &nb) {
        uint8_t *cur = lds + (kt & 1) * STAGE;
        uint8_t *nxt = lds + ((kt + 1) & 1) * STAGE;
        const int64_t kn = (int64_t)(kt + PF) * GEMM_BK;
        if (PF == 2 || kt + 1 < nk) {
            ra.load(kn, p.K);
            rb.load(kn, p.K);
        }
        const uint8_t *as = cur, *bs = cur + BM * GEMM_BK;
        v8i af[TM];
#pragma unroll
        for (int i = 0; i < TM; ++i) af[i] = load_frag(as, wm0 + i * 16 + lr, g);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const v8i bf = load_frag(bs, wn0 + j * 16 + lr, g);
#pragma unroll
            for (int i = 0; i < TM; ++i) MMA::run(acc[i][j], af[i], bf);
        }
        if (kt + 1 < nk) {
            na.store(nxt);
            nb.store(nxt + BM * GEMM_BK);
        }
        __syncthreads();
    };
    if constexpr (PF == 2) {
        for (int kt = 0; kt < nk; kt += 2) {
            step(kt, sa0, sb0, sa1, sb1);
            if (kt + 1 < nk) step(kt + 1, sa1, sb1, sa0, sb0);
        }
    } else {
        for (int kt = 0; kt < nk; ++kt) step(kt, sa0, sb0, sa0, sb0);
    }

    epilogue_tile<MMA, TM, TN, WN>(p, lds, red, acc, m0 + wm0, n0 + wn0, wave, lane);
}

template <int AF, int BF, bool A_MN, bool B_MN, int BM, int BN, int MINW, bool FAST, int PF>
hipError_t launch_tile(GemmParams p, hipStream_t s)
{
    p.tiles_m = (int)((p.M + BM - 1) / BM);
    p.tiles_n = (int)((p.N + BN - 1) / BN);
    if (p.tiles_m == 0 || p.tiles_n == 0) {
        // Empty output: one workgroup whose tile lies wholly outside it
        // (every load reads zeros, no store happens); it still publishes
        // out_amax = 0.
        p.tiles_m = p.tiles_n = 1;
    }
    const int64_t grid = (int64_t)p.tiles_m * p.tiles_n;
    const unsigned batch = p.batch > 1 ? (unsigned)p.batch : 1u;
    p.amax_part = gemm_amax_parts(p.amax_part, grid * batch);
    hipLaunchKernelGGL((qgemm_kernel<AF, BF, A_MN, B_MN, BM, BN, MINW, FAST, PF>), dim3((unsigned)grid, batch),
                       dim3(GEMM_THREADS), 0, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || !p.out_amax || !p.amax_part) return e;
    return launch_amax_finalize(p, grid * batch, s);
}

// Tile size (general kernel): 256 x 256 when that still gives at least two
// tiles per CU, else the largest of 128 x 128, 128 x 64 and 64 x 64 that
// gives one per CU (unaligned operands: 128 x 128).  p.fast selects the
// branch-free buffer-load staging.
template <int AF, int BF> hipError_t launch_nt(GemmParams p, hipStream_t s);
template <int AF, int BF, bool A_MN, bool B_MN, int BM, int BN, int OCC = 1>
hipError_t launch_pipe(GemmParams p, hipStream_t s);
template <int AF, int BF, bool A_MN, bool B_MN, int BM, int BN, int STAGES, int MINW>
hipError_t launch_dl(GemmParams p, hipStream_t s);

template <int AF, int BF, bool A_MN, bool B_MN>
hipError_t launch_layout(const GemmParams &p, hipStream_t s)
{
    if constexpr (A_MN || B_MN) {
        if (!p.fast) return launch_tile<AF, BF, A_MN, B_MN, 128, 128, 2, false, 1>(p, s);
        // An MN-major operand: the direct-to-LDS kernel (transpose reads).
        // Tiles and ring depth keep two workgroups per CU where the grid
        // allows it (measured on the 2048 x 4096 x 1024 backward products):
        // 128x128 with 4 stages (128 KiB of LDS, one per CU) only when that
        // still gives two tiles per CU, else 128x64 with 3 stages (72 KiB),
        // else 64x64 with 4 stages (64 KiB).
        const int64_t nb = p.batch > 1 ? p.batch : 1;
        const int64_t t128 = ((p.M + 127) / 128) * ((p.N + 127) / 128) * nb;
        const int64_t t128x64 = ((p.M + 127) / 128) * ((p.N + 63) / 64) * nb;
        // A single product that still gives every CU a tile of 256 x 128,
        // 128 x 128 or 128 x 64 (but fewer than two of 128 x 128): the
        // pipelined kernel, largest tile first.
        const int64_t cus = device_cu_count();
        if (p.batch <= 1 && p.K > 0 && t128 < 2 * cus) {
            if (((p.M + 255) / 256) * ((p.N + 127) / 128) >= cus)
                return launch_pipe<AF, BF, A_MN, B_MN, 256, 128>(p, s);
            if (t128 >= cus) return launch_pipe<AF, BF, A_MN, B_MN, 128, 128>(p, s);
            if (t128x64 >= cus) return launch_pipe<AF, BF, A_MN, B_MN, 128, 64>(p, s);
        }
        if (t128 >= 512) return launch_dl<AF, BF, A_MN, B_MN, 128, 128, 4, 1>(p, s);
        if (t128x64 >= 512) return launch_dl<AF, BF, A_MN, B_MN, 128, 64, 3, 1>(p, s);
        return launch_dl<AF, BF, A_MN, B_MN, 64, 64, 4, 2>(p, s);
    } else {
        // Both operands K-major.
        const int64_t big = ((p.M + 255) / 256) * ((p.N + 255) / 256);
        // K-major operands with at least one 256 x 256 tile per CU: the
        // pipelined direct-to-LDS kernel.
        if (p.fast && big >= 256 && p.batch <= 1 && p.K > 0) return launch_nt<AF, BF>(p, s);
        // Fewer 256 x 256 tiles than CUs, but at least one 256 x 128 (or
        // 128 x 128) tile per CU: the pipelined kernel with smaller tiles.
        const int64_t cus = device_cu_count();
        if (p.fast && p.batch <= 1 && p.K > 0) {
            // Two or more 128 x 128 tiles per CU: two workgroups per CU.
            if (((p.M + 127) / 128) * ((p.N + 127) / 128) >= 2 * cus)
                return launch_pipe<AF, BF, A_MN, B_MN, 128, 128, 2>(p, s);
            if (((p.M + 255) / 256) * ((p.N + 127) / 128) >= cus) return launch_pipe<AF, BF, A_MN, B_MN, 256, 128>(p, s);
            if (((p.M + 127) / 128) * ((p.N + 127) / 128) >= cus) return launch_pipe<AF, BF, A_MN, B_MN, 128, 128>(p, s);
            if (((p.M + 127) / 128) * ((p.N + 63) / 64) >= cus) return launch_pipe<AF, BF, A_MN, B_MN, 128, 64>(p, s);
        }
        if (p.fast) {
            // The largest tile that still gives every CU a workgroup (batch
            // items count: they are grid rows).
            const int64_t nb = p.batch > 1 ? p.batch : 1;
            const int64_t t128 = ((p.M + 127) / 128) * ((p.N + 127) / 128) * nb;
            const int64_t t128x64 = ((p.M + 127) / 128) * ((p.N + 63) / 64) * nb;
            if (big * nb >= 512) return launch_tile<AF, BF, A_MN, B_MN, 256, 256, 1, true, 1>(p, s);
            if (t128 >= 256) return launch_tile<AF, BF, A_MN, B_MN, 128, 128, 1, true, 2>(p, s);
            if (t128x64 >= 256) return launch_tile<AF, BF, A_MN, B_MN, 128, 64, 2, true, 2>(p, s);
            return launch_tile<AF, BF, A_MN, B_MN, 64, 64, 2, true, 2>(p, s);
        }
        return launch_tile<AF, BF, A_MN, B_MN, 128, 128, 2, false, 1>(p, s);
    }
}

template <int AF, int BF>
hipError_t launch_formats(const GemmParams &p, int a_mn, int b_mn, hipStream_t s)
{
    if (!a_mn && !b_mn) return launch_layout<AF, BF, false, false>(p, s);
    if (!a_mn && b_mn) return launch_layout<AF, BF, false, true>(p, s);
    if (a_mn && !b_mn) return launch_layout<AF, BF, true, false>(p, s);
    return launch_layout<AF, BF, true, true>(p, s);
}

}  // namespace ql
