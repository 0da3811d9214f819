// qgemm_dl.hpp -- scaled FP8 / INT8 GEMM with direct-to-LDS staging for
// every operand layout (the MN-major products of the backward pass: dX =
// g.W reads W MN-major, dW = g^T.X reads both operands MN-major).
//
//   out[m, n] = (sum_k A[m, k] * B[n, k]) * sa * sb (+ bias[n])
//
// [FP8PY] linear_backward_fp8: the two products take the forward's codes in
// their stored layouts.  The pages' own kernel found the MN-major operand
// loads to be the bottleneck; here no thread touches those bytes on their
// way to LDS:
//   * Global -> LDS by buffer loads with an LDS destination (16 bytes per
//     lane, 1 KiB per wave instruction), STAGES-deep ring of LDS buffers:
//     step k+STAGES-1 is in flight while step k is computed.
//   * A K-major operand is stored as the general kernel stores it (rows of
//     128 k-bytes, chunk swizzle lds_swz) and read with ds_read_b128.
//   * An MN-major operand is stored as it lies in memory, one row per k
//     (R mn-bytes, R = tile rows), with its 16-byte chunks XOR-swizzled by a
//     function of k (mn_swz), and read with ds_read_b64_tr_b8 as
//     load_frag_tr in qgemm_impl.hpp describes: 8 k at a time, 4 reads per
//     16x16x128 fragment.
//   * Matrix cores, tile shape, epilogue and tile order as the general kernel
//     (v_mfma_f32_16x16x128_f8f6f4, or paired i8 16x16x64).
// Requirements (checked on the host, p.fast): 16-byte aligned operands and
// leading dimensions, K % 16 == 0 for K-major and MN % 16 == 0 for MN-major
// operands, byte offsets below 2^31.  Rows of a K-major operand past M (N)
// and k-rows of an MN-major operand past K fall outside the buffer range and
// read as zeros; K-major chunks past K are sent outside it.  An MN-major
// tile may read bytes of columns past M (N) inside the buffer; they only
// reach accumulator rows that are never stored.
#pragma once

#include "qgemm_impl.hpp"

namespace ql {

typedef __attribute__((address_space(3))) void *dl_lds_ptr_t;

// One operand of one k-step: R rows (tile rows) x 128 k.  R/32 direct loads
// per wave; load j of wave w fills bytes [(4j + w) * 1024, +1024) of the
// operand's part of a stage.
template <int R, bool MN> struct DlOperand {
    static constexpr int LOADS = R / 32;
    __amdgpu_buffer_rsrc_t rsrc;
    uint32_t off[LOADS];        // tile-relative byte offset of this lane's chunk at k = 0
    int kc[LOADS];              // K-major: this lane's k offset within a step
    uint32_t ld32;
    __device__ __forceinline__ void init(const uint8_t *base, int64_t ld, int64_t row0, int64_t rows_total,
                                         int64_t K, int wave, int lane)
    {
        ld32 = (uint32_t)ld;
        if constexpr (!MN) {
            const int64_t rows_left = rows_total - row0;
            const int64_t bytes = rows_left > 0 ? rows_left * ld : 0;
            rsrc = __builtin_amdgcn_make_buffer_rsrc((void *)(base + row0 * ld), (short)0,
                                                     (int)(bytes < 0x7FFFFFFF ? bytes : 0x7FFFFFFF), BUF_WORD3);
        } else {
            // k-rows >= K fall outside.  A tile wholly past the MN extent
            // (an empty operand, which may have no memory at all) reads
            // nothing.
            const int64_t bytes = row0 < rows_total ? K * ld - row0 : 0;
            rsrc = __builtin_amdgcn_make_buffer_rsrc((void *)(base + row0), (short)0,
                                                     (int)(bytes > 0 ? (bytes < 0x7FFFFFFF ? bytes : 0x7FFFFFFF) : 0),
                                                     BUF_WORD3);
        }
#pragma unroll
        for (int j = 0; j < LOADS; ++j) {
            const int L = (j * 4 + wave) * 1024 + lane * 16;      // this lane's LDS byte in the operand part
            if constexpr (!MN) {
                const int row = L >> 7, pos = (L >> 4) & 7;
                const int c = pos ^ lds_swz(row);
                kc[j] = c * 16;
                off[j] = (uint32_t)(row * ld + c * 16);
            } else {
                const int kr = L / R, pos = (L % R) >> 4;
                const int c = pos ^ mn_swz<R>(kr);
                kc[j] = 0;
                off[j] = (uint32_t)(kr * ld + c * 16);
            }
        }
    }
    // Issue this wave's loads of the step at k offset k0 into `part` (the
    // operand's part of a stage, wave-uniform LDS byte address).
    __device__ __forceinline__ void issue(uint32_t part, int wave, int64_t k0, int64_t K) const
    {
#pragma unroll
        for (int j = 0; j < LOADS; ++j) {
            uint32_t o;
            if constexpr (!MN) o = k0 + kc[j] < K ? off[j] + (uint32_t)k0 : BUF_OOB;
            else o = off[j] + (uint32_t)k0 * ld32;
            const dl_lds_ptr_t dst = (dl_lds_ptr_t)(uintptr_t)(part + (uint32_t)(j * 4 + wave) * 1024u);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 16, (int)o, 0, 0, 0);
        }
    }
};

// LDS reads as inline assembly.  The compiler sees no LDS access here, so it
// does not make them wait for the direct loads still in flight (it cannot
// tell which stage they write); completion is awaited explicitly with
// lgkmcnt, and the destination registers are tied to that wait so that no
// use is scheduled before it.

__device__ __forceinline__ u32x4 dl_read_b128(uint32_t addr)
{
    u32x4 x;
    asm volatile("ds_read_b128 %0, %1" : "=v"(x) : "v"(addr) : "memory");
    return x;
}

__device__ __forceinline__ u32x2 dl_read_tr8(uint32_t addr)
{
    u32x2 x;
    asm volatile("ds_read_b64_tr_b8 %0, %1" : "=v"(x) : "v"(addr) : "memory");
    return x;
}

template <int N> __device__ __forceinline__ void dl_lgkm_wait()
{
    static_assert(N >= 0 && N < 16, "lgkmcnt");
    asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N) : "memory");
}

template <typename T> __device__ __forceinline__ void dl_tie(T &x) { asm volatile("" : "+v"(x)); }

// Compile-time loop: f(integral_constant<int, I>) for I in [B, E).
template <int B, int E, typename F> __device__ __forceinline__ void dl_unroll(F &&f)
{
    if constexpr (B < E) {
        f(std::integral_constant<int, B>());
        dl_unroll<B + 1, E>(f);
    }
}

// One 16 x 128 operand fragment in flight: K-major as two 16-byte reads
// (k = 32 (l >> 4) + 0..15, +16..31 of row l & 15), MN-major as four
// transpose reads of 8 k each.
template <bool MN> struct DlFrag;
template <> struct DlFrag<false> {
    static constexpr int READS = 2;
    u32x4 h[2];
    __device__ __forceinline__ void read(uint32_t base, const uint32_t (&off)[4])
    {
        h[0] = dl_read_b128(base + off[0]);
        h[1] = dl_read_b128(base + off[1]);
    }
    __device__ __forceinline__ void tie() { dl_tie(h[0]); dl_tie(h[1]); }
    __device__ __forceinline__ v8i get() const
    {
        return v8i{(int)h[0].x, (int)h[0].y, (int)h[0].z, (int)h[0].w, (int)h[1].x, (int)h[1].y, (int)h[1].z, (int)h[1].w};
    }
};
template <> struct DlFrag<true> {
    static constexpr int READS = 4;
    u32x2 q[4];
    __device__ __forceinline__ void read(uint32_t base, const uint32_t (&off)[4])
    {
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = dl_read_tr8(base + off[i]);
    }
    __device__ __forceinline__ void tie()
    {
#pragma unroll
        for (int i = 0; i < 4; ++i) dl_tie(q[i]);
    }
    __device__ __forceinline__ v8i get() const
    {
        return v8i{(int)q[0].x, (int)q[0].y, (int)q[1].x, (int)q[1].y, (int)q[2].x, (int)q[2].y, (int)q[3].x, (int)q[3].y};
    }
};

// This lane's byte offsets (within an operand part) of the reads of the
// fragment whose first tile row is row0.  K-major: chunks 2(l>>4), +1 of row
// row0 + (l & 15) in the general kernel's swizzled layout.  MN-major
// (k-rows of R bytes): lanes 2j, 2j+1 of a 16-lane block address k-row
// 32 (l>>4) + 8q + j, mn bytes [row0, row0+8) and [row0+8, row0+16).
template <int R, bool MN>
__device__ __forceinline__ void dl_frag_offsets(int row0, int lane, uint32_t (&off)[4])
{
    if constexpr (!MN) {
        const int row = row0 + (lane & 15), g = lane >> 4;
        off[0] = (uint32_t)lds_off(row, 2 * g);
        off[1] = (uint32_t)lds_off(row, 2 * g + 1);
        off[2] = off[3] = 0;
    } else {
        const int b = lane >> 4, t = lane & 15;
        const int c = row0 >> 4, h = t & 1;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int kr = 32 * b + 8 * q + (t >> 1);
            off[q] = (uint32_t)(kr * R + ((c ^ mn_swz<R>(kr)) << 4) + 8 * h);
        }
    }
}

template <int AF, int BF, bool A_MN, bool B_MN, int BM, int BN, int STAGES, int MINW>
__global__ __launch_bounds__(GEMM_THREADS, MINW) void qgemm_dl_kernel(GemmParams p)
{
    typedef Mma<AF, BF> MMA;
    typedef typename MMA::acc_t acc_t;
    constexpr int WM = BM / 2, WN = BN / 2, TM = WM / 16, TN = WN / 16;
    constexpr int A_BYTES = BM * GEMM_BK, STAGE = (BM + BN) * GEMM_BK;
    static_assert(STAGES >= 2, "ring depth");
    __shared__ __attribute__((aligned(16))) uint8_t lds[STAGES * STAGE];
    __shared__ uint32_t red[GEMM_THREADS / 64];

    select_batch_item(p);
    int tm, tn;
    tile_coords(p.tiles_m, p.tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm0 = (wave >> 1) * WM, wn0 = (wave & 1) * WN;

    DlOperand<BM, A_MN> opa;
    DlOperand<BN, B_MN> opb;
    opa.init(p.a, p.lda, m0, p.M, p.K, wave, lane);
    opb.init(p.b, p.ldb, n0, p.N, p.K, wave, lane);
    constexpr int LOADS = DlOperand<BM, A_MN>::LOADS + DlOperand<BN, B_MN>::LOADS;   // per wave per step

    const uint32_t lds_base = (uint32_t)(uintptr_t)(dl_lds_ptr_t)lds;
    auto issue_step = [&](int step) {
        const uint32_t st = lds_base + (uint32_t)((step % STAGES) * STAGE);
        const int64_t k0 = (int64_t)step * GEMM_BK;
        opa.issue(st, wave, k0, p.K);
        opb.issue(st + A_BYTES, wave, k0, p.K);
    };

    acc_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = acc_t{0, 0, 0, 0};

    uint32_t offa[TM][4], offb[TN][4];
#pragma unroll
    for (int i = 0; i < TM; ++i) dl_frag_offsets<BM, A_MN>(wm0 + i * 16, lane, offa[i]);
#pragma unroll
    for (int j = 0; j < TN; ++j) dl_frag_offsets<BN, B_MN>(wn0 + j * 16, lane, offb[j]);

    const int nk = (int)((p.K + GEMM_BK - 1) / GEMM_BK);
    // Prologue: steps 0 .. STAGES-2 in flight (steps past the end load
    // zeros or nothing that is read).
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
        if (s < nk) issue_step(s);

    for (int kt = 0; kt < nk; ++kt) {
        // Wait for this wave's loads of step kt (later steps may stay in
        // flight), then for every wave's: the barrier also means that every
        // wave is done with step kt-1, whose buffer the next refill takes.
        const int ahead = nk - 1 - kt < STAGES - 2 ? nk - 1 - kt : STAGES - 2;   // steps issued after kt
        dl_unroll<0, STAGES - 1>([&](auto A) {
            constexpr int n = decltype(A)::value * LOADS;   // vmcnt(ahead * LOADS)
            static_assert(n < 64, "vmcnt holds 6 bits");
            if (ahead == decltype(A)::value) __builtin_amdgcn_s_waitcnt(0x0F70 | (n & 0xF) | ((n >> 4) << 14));
        });
        // A bare barrier: a fenced one would also wait for the later steps'
        // loads.  Every wave's reads of step kt-1 are complete here (the
        // matrix cores consumed them).
        __builtin_amdgcn_s_barrier();
        if (kt + STAGES - 1 < nk) issue_step(kt + STAGES - 1);

        // All fragment reads of the step, then the matrix cores column by
        // column of fragments, each after the reads it needs (LDS reads
        // complete in order).
        const uint32_t as = lds_base + (uint32_t)((kt % STAGES) * STAGE), bs = as + A_BYTES;
        DlFrag<A_MN> fa[TM];
        DlFrag<B_MN> fb[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) fa[i].read(as, offa[i]);
#pragma unroll
        for (int j = 0; j < TN; ++j) fb[j].read(bs, offb[j]);
        constexpr int RB = DlFrag<B_MN>::READS;
        dl_lgkm_wait<(TN - 1) * RB>();
#pragma unroll
        for (int i = 0; i < TM; ++i) fa[i].tie();
        v8i av[TM];
#pragma unroll
        for (int i = 0; i < TM; ++i) av[i] = fa[i].get();
        dl_unroll<0, TN>([&](auto J) {
            constexpr int j = decltype(J)::value;
            if constexpr (j > 0) dl_lgkm_wait<(TN - 1 - j) * RB>();
            fb[j].tie();
            const v8i bv = fb[j].get();
#pragma unroll
            for (int i = 0; i < TM; ++i) MMA::run(acc[i][j], av[i], bv);
            __builtin_amdgcn_sched_barrier(0);      // keep each column's matrix ops before the next wait
        });
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);
    epilogue_tile<MMA, TM, TN, WN>(p, lds, red, acc, m0 + wm0, n0 + wn0, wave, lane);
}

template <int AF, int BF, bool A_MN, bool B_MN, int BM, int BN, int STAGES, int MINW>
hipError_t launch_dl(GemmParams p, hipStream_t s)
{
    p.tiles_m = (int)((p.M + BM - 1) / BM);
    p.tiles_n = (int)((p.N + BN - 1) / BN);
    if (p.tiles_m == 0 || p.tiles_n == 0) p.tiles_m = p.tiles_n = 1;   // as launch_tile: out_amax = 0
    const int64_t grid = (int64_t)p.tiles_m * p.tiles_n;
    const unsigned batch = p.batch > 1 ? (unsigned)p.batch : 1u;
    p.amax_part = gemm_amax_parts(p.amax_part, grid * batch);
    hipLaunchKernelGGL((qgemm_dl_kernel<AF, BF, A_MN, B_MN, BM, BN, STAGES, MINW>), dim3((unsigned)grid, batch),
                       dim3(GEMM_THREADS), 0, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || !p.out_amax || !p.amax_part) return e;
    return launch_amax_finalize(p, grid * batch, s);
}

}  // namespace ql
