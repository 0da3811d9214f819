// qgemm_nt.hpp -- pipelined scaled GEMM for K-major A and B (the "NT"
// forward product out = A @ B^T of AstrAI ops/fp8.py mm_fp8 /
// linear_forward_fp8, with B the [N, K] weight), gfx950.
//
// One workgroup of 4 waves computes a 256 x 256 output tile; each wave owns
// a 128 x 128 quarter as 4 x 4 blocks of v_mfma_f32_32x32x64_f8f6f4 (FP8,
// per-operand formats) or pairs of v_mfma_i32_32x32x32_i8 (INT8).
//
// K advances 128 bytes per step -- whole 128-byte cache lines of every row
// -- through 2 LDS stages of 64 KiB (256 rows of A and of B, 128 bytes per
// row).  Global data goes straight into LDS with buffer_load_dwordx4 ...
// lds (no registers, no LDS write instructions).  A step is worked in two
// 64-deep halves with two fragment register sets: half 0's MFMAs run while
// half 1's fragments are read; then this wave is done with the stage, and
// after the barrier (which also certifies everyone's loads of the next
// step) half 1's MFMAs run while the next step's first fragments are read
// and the freed stage is refilled with the step after next.  With one wave
// per SIMD the program order is the schedule, so every MFMA slot carries
// one LDS read and, early in half 1, two loads.  Every step has the same
// shape: steps past the end load zeros (offsets past K are out of the
// buffer range) into a stage nobody reads.  Rows past M / N and chunks
// past K come back as zeros through the buffer range check.
//
// LDS rows are 128 bytes = 8 chunks of 16 bytes; chunk c of row r sits at
// position c ^ f(r), f(r) = g((r >> 1) & 7) ^ (((r >> 4) & 1) << 2), g
// swapping bits 1 and 2.  A 16-byte LDS read serves 16 lanes per clock on
// gfx950; with this f every 16-lane group of a fragment read (lanes 0-15,
// or 0-7 with 32-39, or 0-3/16-19/32-35/48-51, or 0-3/8-11/16-19/24-27)
// touches 16 distinct bank quads.  A direct-to-LDS load writes lane i's 16
// bytes at position i of the wave's 1 KiB window, so each lane fetches the
// global chunk that belongs there.
//
// The matrix cores compute the transposed tile C^T = B A^T (B's fragment
// as the first operand): then each lane's register quad holds 4
// consecutive output columns of one row, which the epilogue moves through
// LDS with 16-byte writes.
#pragma once

#include "qgemm_impl.hpp"

namespace ql {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int NT_BM = 256, NT_BN = 256, NT_BK = 128, NT_STAGES = 2;
constexpr int NT_CHUNKS = NT_BK / 16;                             // 16-byte chunks per row (8)
constexpr int NT_STAGE_BYTES = (NT_BM + NT_BN) * NT_BK;          // 64 KiB
constexpr int NT_LOADS = NT_STAGE_BYTES / (GEMM_THREADS * 16);   // 16-byte loads per thread per step (16)

__device__ __forceinline__ int nt_swz(int r)
{
    const int m = (r >> 1) & 7;
    const int g = (m & 1) | ((m & 2) << 1) | ((m & 4) >> 1);
    return g ^ (((r >> 4) & 1) << 2);
}

template <int AF, int BF> struct Mma32 {
    typedef v16f acc_t;
    static constexpr bool INT_ACC = false;
    __device__ __forceinline__ static void run(acc_t &c, const v8i &a, const v8i &b)
    {
        c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, AF, BF, 0, 0, 0, 0);
    }
    __device__ __forceinline__ static uint32_t bits(const acc_t &c, int r) { return __float_as_uint(c[r]); }
};

template <> struct Mma32<FMT_INT8, FMT_INT8> {
    typedef v16i acc_t;
    static constexpr bool INT_ACC = true;
    __device__ __forceinline__ static void run(acc_t &c, const v8i &a, const v8i &b)
    {
        v4i a0 = {a[0], a[1], a[2], a[3]}, a1 = {a[4], a[5], a[6], a[7]};
        v4i b0 = {b[0], b[1], b[2], b[3]}, b1 = {b[4], b[5], b[6], b[7]};
        c = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, b0, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, b1, c, 0, 0, 0);
    }
    __device__ __forceinline__ static uint32_t bits(const acc_t &c, int r) { return (uint32_t)c[r]; }
};

// 32 rows x 64 k fragment for lane l: row (l & 31), k = 64*half +
// 32*(l >> 5) .. +31 (logical chunks 4*half + 2*(l >> 5) and the next).
// The two 16-byte LDS reads are issued as inline assembly: the compiler's
// wait insertion cannot tell that they never touch a stage a direct-to-LDS
// load is still filling, and would otherwise wait for every load in flight
// before each read.  Completion is awaited explicitly (nt_wait_lgkm) before
// the fragments are used.
__device__ __forceinline__ uint32_t nt_frag_addr(uint32_t lds_base, int row, int chunk)
{
    return lds_base + (uint32_t)(row * NT_BK + ((chunk ^ nt_swz(row)) << 4));
}

__device__ __forceinline__ u32x4 nt_read16(uint32_t addr)
{
    u32x4 x;
    asm volatile("ds_read_b128 %0, %1" : "=v"(x) : "v"(addr) : "memory");
    return x;
}

typedef __attribute__((address_space(3))) void *lds_ptr_t;

// Wait for all LDS reads of this wave; the 16 fragment halves just read are
// tied to the wait so no use can move above it.
__device__ __forceinline__ void nt_wait_parts(u32x4 (&v)[16])
{
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7]),
                   "+v"(v[8]), "+v"(v[9]), "+v"(v[10]), "+v"(v[11]), "+v"(v[12]), "+v"(v[13]), "+v"(v[14]), "+v"(v[15])
                 :
                 : "memory");
}

__device__ __forceinline__ v8i nt_join(const u32x4 &x, const u32x4 &y)
{
    return __builtin_shufflevector((v4i)x, (v4i)y, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <int AF, int BF>
__global__ __launch_bounds__(GEMM_THREADS, 1) void qgemm_nt_kernel(GemmParams p)
{
    typedef Mma32<BF, AF> MMA;                 // operands swapped: acc holds C^T
    typedef typename MMA::acc_t acc_t;
    constexpr int WM = NT_BM / 2, WN = NT_BN / 2, TM = WM / 32, TN = WN / 32;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[NT_STAGES * NT_STAGE_BYTES];
    __shared__ uint32_t red[GEMM_THREADS / 64];

    int tm, tn;
    tile_coords(p.tiles_m, p.tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * NT_BM, n0 = (int64_t)tn * NT_BN;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar LDS windows
    const int wm0 = (wave >> 1) * WM, wn0 = (wave & 1) * WN;

    // Buffer resources from the tile's first row; rows past the matrix are
    // outside num_records and load as zeros.
    const int64_t a_rows = p.M - m0, b_rows = p.N - n0;
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(p.a + m0 * p.lda), (short)0, (int)(a_rows > 0 ? a_rows * p.lda : 0), BUF_WORD3);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(p.b + n0 * p.ldb), (short)0, (int)(b_rows > 0 ? b_rows * p.ldb : 0), BUF_WORD3);

    // Load j of this wave covers stage bytes [(jj*4 + wave) * 1024, +1024)
    // of the A half (j < NT_LOADS/2, jj = j) or the B half (jj = j -
    // NT_LOADS/2).  Lane i lands at position q = (jj*4 + wave)*64 + i
    // (16-byte units): row q/8, swizzled chunk q%8, so it fetches logical
    // chunk (q%8) ^ f(row).
    uint32_t goff[NT_LOADS];
    int kchunk[NT_LOADS];
#pragma unroll
    for (int j = 0; j < NT_LOADS; ++j) {
        const int q = ((j % (NT_LOADS / 2)) * 4 + wave) * 64 + lane;
        const int row = q / NT_CHUNKS;
        const int c = (q % NT_CHUNKS) ^ nt_swz(row);
        kchunk[j] = c * 16;
        goff[j] = (uint32_t)(row * (j < NT_LOADS / 2 ? p.lda : p.ldb) + c * 16);
    }

    const int K32 = (int)p.K;
    // Direct-to-LDS load j (0 .. NT_LOADS-1) of `step`.  Chunks past K (only
    // in a partial last step) get an offset outside the buffer range.
    auto issue_one = [&](int step, int j) {
        uint8_t *st = lds + (step % NT_STAGES) * NT_STAGE_BYTES;
        const int k0 = step * NT_BK;
        const bool is_a = j < NT_LOADS / 2;
        const int win = ((j % (NT_LOADS / 2)) * 4 + wave) * 1024 + (is_a ? 0 : NT_BM * NT_BK);
        uint32_t off = goff[j] + (uint32_t)k0;
        if (k0 + NT_BK > K32) off = k0 + kchunk[j] < K32 ? off : BUF_OOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(is_a ? ra : rb, (lds_ptr_t)(st + win), 16, (int)off, 0, 0, 0);
    };
    auto issue = [&](int step) {
#pragma unroll
        for (int j = 0; j < NT_LOADS; ++j) issue_one(step, j);
    };

    acc_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = acc_t{};

    const int nk = (int)((p.K + NT_BK - 1) / NT_BK);
    const int lr = lane & 31, h = lane >> 5;
    const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_ptr_t)lds;

    // LDS address of fragment half t (0..15) of one 64-deep half of `step`:
    // t/2 selects A fragment 0..3 or B fragment 0..3, t%2 the 16-byte half.
    auto frag_addr = [&](int step, int half, int t) {
        const uint32_t as = lds_base + (uint32_t)((step % NT_STAGES) * NT_STAGE_BYTES);
        const int f = t >> 1;
        const int chunk = 4 * half + 2 * h + (t & 1);
        return f < TM ? nt_frag_addr(as, wm0 + f * 32 + lr, chunk)
                      : nt_frag_addr(as + NT_BM * NT_BK, wn0 + (f - TM) * 32 + lr, chunk);
    };
    auto join = [&](u32x4 (&pt)[16], v8i (&af)[TM], v8i (&bf)[TN]) {
#pragma unroll
        for (int i = 0; i < TM; ++i) af[i] = nt_join(pt[2 * i], pt[2 * i + 1]);
#pragma unroll
        for (int j = 0; j < TN; ++j) bf[j] = nt_join(pt[2 * (TM + j)], pt[2 * (TM + j) + 1]);
    };
    constexpr int VM_ONE_STEP = 0x0F70 | (NT_LOADS & 0xF) | ((NT_LOADS >> 4) << 14);
    v8i fa0[TM], fb0[TN], fa1[TM], fb1[TN];
    u32x4 pt[16];
    if (nk > 0) {
        issue(0);
        issue(1);
        __builtin_amdgcn_s_waitcnt(VM_ONE_STEP);
        __builtin_amdgcn_s_barrier();
#pragma unroll
        for (int t = 0; t < 16; ++t) pt[t] = nt_read16(frag_addr(0, 0, t));
        nt_wait_parts(pt);
        join(pt, fa0, fb0);
    }
    for (int kt = 0; kt < nk; ++kt) {
        // Half 0: MFMAs on set 0, read half 1 into set 1.
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            MMA::run(acc[t >> 2][t & 3], fb0[t & 3], fa0[t >> 2]);
            pt[t] = nt_read16(frag_addr(kt, 1, t));
            __builtin_amdgcn_sched_barrier(0);
        }
        nt_wait_parts(pt);
        join(pt, fa1, fb1);
        // This wave is done with stage kt; everyone's loads of step kt+1
        // have landed once all waves pass the barrier.
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __builtin_amdgcn_s_barrier();
        // Half 1: MFMAs on set 1, read step kt+1's half 0 into set 0, and
        // refill stage kt with step kt+2 (two loads per slot, early).
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            MMA::run(acc[t >> 2][t & 3], fb1[t & 3], fa1[t >> 2]);
            pt[t] = nt_read16(frag_addr(kt + 1, 0, t));
            if (t < NT_LOADS / 2) {
                issue_one(kt + 2, 2 * t);
                issue_one(kt + 2, 2 * t + 1);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        nt_wait_parts(pt);
        join(pt, fa0, fb0);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();

    // Epilogue through LDS, one 32-row slab of the wave tile at a time.
    // Block (i, j) holds C^T: element r of lane l is output row i*32 + l%32,
    // column j*32 + (r/4)*8 + 4*(l/32) + r%4, so register quad q goes to LDS
    // as one 16-byte write; then each lane takes 4 consecutive columns of a
    // row for the fused epilogue and a contiguous store.
    constexpr int EP_LD = WN + 4;                        // padded row, in words
    uint32_t *ep = reinterpret_cast<uint32_t *>(lds) + wave * 32 * EP_LD;
    Epilogue epi(p);
    uint32_t vmax = 0;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        __syncthreads();
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *reinterpret_cast<uint4 *>(ep + lr * EP_LD + j * 32 + q * 8 + h * 4) =
                    make_uint4(MMA::bits(acc[i][j], 4 * q), MMA::bits(acc[i][j], 4 * q + 1),
                               MMA::bits(acc[i][j], 4 * q + 2), MMA::bits(acc[i][j], 4 * q + 3));
        __syncthreads();
        constexpr int C4 = WN / 4;
#pragma unroll 1
        for (int idx = lane; idx < 32 * C4; idx += 64) {
            const int rr = idx / C4, c4 = idx - rr * C4;
            const uint4 w = *reinterpret_cast<const uint4 *>(ep + rr * EP_LD + c4 * 4);
            const int64_t row = m0 + wm0 + i * 32 + rr;
            const int64_t col = n0 + wn0 + c4 * 4;
            if (row < p.M && col < p.N) vmax = epi.store4<MMA::INT_ACC>(w, row, col, vmax);
        }
    }
    if (p.out_amax) {
        vmax = block_max_u32(vmax, red);
        if (threadIdx.x == 0) {
            uint32_t bits;
            if (elect_last_max(p.ws, vmax, &bits)) p.out_amax[0] = __uint_as_float(bits);
        }
    }
}

template <int AF, int BF>
hipError_t launch_nt(GemmParams p, hipStream_t s)
{
    p.tiles_m = (int)((p.M + NT_BM - 1) / NT_BM);
    p.tiles_n = (int)((p.N + NT_BN - 1) / NT_BN);
    const int64_t grid = (int64_t)p.tiles_m * p.tiles_n;
    hipLaunchKernelGGL((qgemm_nt_kernel<AF, BF>), dim3((unsigned)grid), dim3(GEMM_THREADS), 0, s, p);
    return hipGetLastError();
}

}  // namespace ql
