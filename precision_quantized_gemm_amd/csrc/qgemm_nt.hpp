// qgemm_nt.hpp -- pipelined scaled GEMM for K-major A and B (the "NT"
// forward product out = A @ B^T of AstrAI ops/fp8.py mm_fp8 /
// linear_forward_fp8, with B the [N, K] weight), gfx950.
//
// One workgroup of 4 waves computes a 256 x 256 output tile; each wave owns
// a 128 x 128 quarter as 4 x 4 blocks of v_mfma_f32_32x32x64_f8f6f4 (FP8,
// per-operand formats; INT8 as two v_mfma_i32_32x32x32_i8 per block).
//
// K advances 128 bytes per step -- whole 128-byte cache lines of every row
// -- through 2 LDS stages of 64 KiB (256 rows of A and of B, 128 bytes per
// row).  Global data goes straight into LDS with buffer_load_dwordx4 ...
// lds (no registers, no LDS write instructions).  A step is worked in two
// 64-deep halves with two fragment register sets: half 0's MFMAs run while
// half 1's fragments are read; once every wave holds them (a barrier part
// way through half 0) the stage is refilled with the step after next, one
// load per MFMA slot into half 1; after the mid-step barrier (which
// certifies everyone's loads of the next step) half 1's MFMAs run while the
// next step's first fragments are read.  With one wave per SIMD the program
// order is the schedule: every MFMA slot carries up to two LDS reads and
// one load.  Every step has the same
// shape: steps past the end load zeros (offsets past K are out of the
// buffer range) into a stage nobody reads.  Rows past M / N and chunks
// past K come back as zeros through the buffer range check.
//
// LDS rows are 128 bytes = 8 chunks of 16 bytes; chunk c of row r sits at
// position c ^ f(r), f(r) = (r >> 1) & 7.  A 16-byte LDS read is served 16
// lanes per clock from 64 banks of 4 bytes, so 16 lanes that share a clock
// must hit 16 distinct 16-byte slots of a 256-byte bank line.  Which lanes
// share a clock is not simply lanes 0-15, 16-31, ...; this f was chosen
// because the hardware's bank-conflict counter reads zero for all four
// fragment read shapes below (rows r..r+31, chunk pairs c and c+2), and it
// also is conflict-free under the plain consecutive grouping.  A
// direct-to-LDS load writes lane i's 16 bytes at position i of the wave's
// 1 KiB window, so each lane fetches the global chunk that belongs there.
//
// The matrix cores compute the transposed tile C^T = B A^T (B's fragment
// as the first operand): then each lane's register quad holds 4
// consecutive output columns of one row, which the epilogue moves through
// LDS with 16-byte writes.
//
// The grid is persistent (CHAIN) when every tile is whole, every epilogue
// stays in registers (per-tensor scales or raw INT32 output, 16-byte
// aligned rows) and K is an even number of whole steps: one workgroup per
// CU walks tiles id, id + grid, ...  The two refills past a tile's last
// step fetch the next tile's first two steps instead of nothing, and the
// last step reads the next tile's first fragments, so the next tile's
// start-up latency hides behind this tile's epilogue and no workgroup
// launch separates the two.  Other shapes take one tile per workgroup.
#pragma once

#include "qgemm_common.hpp"

namespace ql {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int NT_BM = 256, NT_BN = 256, NT_BK = 128, NT_STAGES = 2;
constexpr int NT_CHUNKS = NT_BK / 16;                             // 16-byte chunks per row (8)
constexpr int NT_STAGE_BYTES = (NT_BM + NT_BN) * NT_BK;          // 64 KiB
constexpr int NT_LOADS = NT_STAGE_BYTES / (GEMM_THREADS * 16);   // 16-byte loads per thread per step (16)
constexpr int NT_A_BYTES = NT_BM * NT_BK;                        // one stage of A (or B): 32 KiB
constexpr int NT_READS_PER_SLOT = 2;  // fragment reads issued per MFMA slot (front-loaded)
// Refill schedule: the step-after-next's NT_LOADS loads go out
// NT_LOADS_PER_SLOT per MFMA slot from slot NT_LOAD_SLOT0, counted over the
// step's two halves (0-15 the first, 16-31 the second).  A start in the
// first half adds a barrier there, once every wave has read the stage.
constexpr int NT_LOAD_SLOT0 = 10;
constexpr int NT_LOADS_PER_SLOT = 1;
static_assert(NT_LOAD_SLOT0 >= 16 || NT_LOAD_SLOT0 * NT_READS_PER_SLOT >= 16,
              "the refill starts only after this wave has issued every read of the stage");
static_assert(NT_LOAD_SLOT0 + (NT_LOADS + NT_LOADS_PER_SLOT - 1) / NT_LOADS_PER_SLOT <= 32,
              "the refill ends within the step");
// Refill loads issued before the mid-step wait, which may stay in flight.
constexpr int NT_REFILL_EARLY =
    NT_LOAD_SLOT0 >= 16 ? 0
                        : ((16 - NT_LOAD_SLOT0) * NT_LOADS_PER_SLOT < NT_LOADS ? (16 - NT_LOAD_SLOT0) * NT_LOADS_PER_SLOT
                                                                                : NT_LOADS);
constexpr int NT_VM_MID = 0x0F70 | (NT_REFILL_EARLY & 0xF) | ((NT_REFILL_EARLY >> 4) << 14);

__device__ __forceinline__ int nt_swz(int r) { return (r >> 1) & 7; }

template <int AF, int BF> struct Mma32 {
    typedef v16f acc_t;
    static constexpr bool INT_ACC = false;
    // a = (a0, a1), b = (b0, b1): each operand's 32 bytes as two 16-byte halves.
    __device__ __forceinline__ static void run(acc_t &c, const u32x4 &a0, const u32x4 &a1, const u32x4 &b0,
                                               const u32x4 &b1)
    {
        const v8i a = __builtin_shufflevector((v4i)a0, (v4i)a1, 0, 1, 2, 3, 4, 5, 6, 7);
        const v8i b = __builtin_shufflevector((v4i)b0, (v4i)b1, 0, 1, 2, 3, 4, 5, 6, 7);
        c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, AF, BF, 0, 0, 0, 0);
    }
    // The same with a zero accumulator in (the first k of a tile): the
    // instruction's inline constant, so no register needs clearing.
    __device__ __forceinline__ static void run0(acc_t &c, const u32x4 &a0, const u32x4 &a1, const u32x4 &b0,
                                                const u32x4 &b1)
    {
        const v8i a = __builtin_shufflevector((v4i)a0, (v4i)a1, 0, 1, 2, 3, 4, 5, 6, 7);
        const v8i b = __builtin_shufflevector((v4i)b0, (v4i)b1, 0, 1, 2, 3, 4, 5, 6, 7);
        c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc_t{}, AF, BF, 0, 0, 0, 0);
    }
    __device__ __forceinline__ static uint32_t bits(const acc_t &c, int r) { return __float_as_uint(c[r]); }
};

// INT8: two v_mfma_i32_32x32x32_i8 per 64-deep fragment pair.  Each takes
// 16 of a lane's 32 bytes (the low halves, then the high ones) from A and B
// alike, so the two cover every k of the pair once; the sum does not depend
// on which k each instruction sees.  The accumulator layout is the FP32
// one's.
template <> struct Mma32<FMT_INT8, FMT_INT8> {
    typedef v16i acc_t;
    static constexpr bool INT_ACC = true;
    __device__ __forceinline__ static void run(acc_t &c, const u32x4 &a0, const u32x4 &a1, const u32x4 &b0,
                                               const u32x4 &b1)
    {
        c = __builtin_amdgcn_mfma_i32_32x32x32_i8((v4i)a0, (v4i)b0, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_i32_32x32x32_i8((v4i)a1, (v4i)b1, c, 0, 0, 0);
    }
    __device__ __forceinline__ static void run0(acc_t &c, const u32x4 &a0, const u32x4 &a1, const u32x4 &b0,
                                                const u32x4 &b1)
    {
        c = __builtin_amdgcn_mfma_i32_32x32x32_i8((v4i)a0, (v4i)b0, acc_t{}, 0, 0, 0);
        c = __builtin_amdgcn_mfma_i32_32x32x32_i8((v4i)a1, (v4i)b1, c, 0, 0, 0);
    }
    __device__ __forceinline__ static uint32_t bits(const acc_t &c, int r) { return (uint32_t)c[r]; }
};


// 32 rows x 64 k fragment for lane l: row (l & 31), k = 64*half +
// 32*(l >> 5) .. +31 (logical chunks 4*half + 2*(l >> 5) and the next).
// The two 16-byte LDS reads are issued as inline assembly: the compiler's
// wait insertion cannot tell that they never touch a stage a direct-to-LDS
// load is still filling, and would otherwise wait for every load in flight
// before each read.  Completion is awaited explicitly (nt_wait_parts) before
// the fragments are used.  The stage and fragment offsets ride in the
// instruction's immediate, so a read needs no address arithmetic.

template <int OFF>
__device__ __forceinline__ u32x4 nt_read16(uint32_t addr)
{
    static_assert(OFF >= 0 && OFF < 65536, "LDS immediate offset is 16 bits");
    u32x4 x;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(x) : "v"(addr), "n"(OFF) : "memory");
    return x;
}

// Compile-time loop: f(integral_constant<int, I>) for I in [B, E).
template <int B, int E, typename F>
__device__ __forceinline__ void nt_unroll(F &&f)
{
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        nt_unroll<B + 1, E>(f);
    }
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


// E4M3 output without bias for 16 consecutive accumulators of one row: the
// codes are the accumulators times RN(sa*sb / out_scale), and out_amax is
// max |acc| times |sa*sb| once per workgroup (rounding is monotone, so that
// is max |RN(acc*sa*sb)|); this keeps max |acc| in macc.
template <bool INT_ACC>
__device__ __forceinline__ uint4 nt_e4m3_codes16(const Epilogue &epi, const uint4 (&w)[4], float &macc)
{
    auto val = [](uint32_t x) { return INT_ACC ? (float)(int32_t)x : __uint_as_float(x); };
    float a[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        a[4 * q + 0] = val(w[q].x); a[4 * q + 1] = val(w[q].y);
        a[4 * q + 2] = val(w[q].z); a[4 * q + 3] = val(w[q].w);
    }
    // max |a| three operands per instruction: five over 15 values, three
    // more folding them, the 16th and the running maximum.
    auto mx3 = [](float x, float y, float z) {
        return __builtin_elementwise_maximum(x, __builtin_elementwise_maximum(y, z));
    };
    float t[5];
#pragma unroll
    for (int g = 0; g < 5; ++g)
        t[g] = mx3(__builtin_fabsf(a[3 * g]), __builtin_fabsf(a[3 * g + 1]), __builtin_fabsf(a[3 * g + 2]));
    float m = mx3(macc, t[0], t[1]);
    m = mx3(m, t[2], t[3]);
    macc = mx3(m, t[4], __builtin_fabsf(a[15]));
    const float s = epi.s_out;
    uint4 c;
    c.x = encode4<FMT_E4M3>(a[0] * s, a[1] * s, a[2] * s, a[3] * s);
    c.y = encode4<FMT_E4M3>(a[4] * s, a[5] * s, a[6] * s, a[7] * s);
    c.z = encode4<FMT_E4M3>(a[8] * s, a[9] * s, a[10] * s, a[11] * s);
    c.w = encode4<FMT_E4M3>(a[12] * s, a[13] * s, a[14] * s, a[15] * s);
    return c;
}

// Position of 16-byte chunk c of row r in a wave's 32-row x 128-byte line
// staging area (the whole-line epilogues): c ^ f(r), the operand stages'
// swizzle.  Writes (lane l: row l % 32, one chunk per half-wave) and reads
// (lane l: row 8k + l / 8, chunk l % 8) then put the 16 lanes of one LDS
// clock on 16 distinct 16-byte bank slots, both when a clock takes the
// lane quads of a half-wave whose quad index has equal parity (how the
// 16-byte reads are served) and when it takes lanes 16i .. 16i+15 (the
// 16-byte writes behave like the latter).  An earlier swizzle here,
// 4 r1 + (r >> 3 & 3), conflicted two-way on the reads and on the writes
// (the bank-conflict counter read 3.7 M cycles per large GEMM).
__device__ __forceinline__ int nt_line_swz(int r) { return nt_swz(r); }

__device__ __forceinline__ void nt_store16_stream(uint8_t *dst, uint4 c)
{
    __builtin_nontemporal_store(u32x4{c.x, c.y, c.z, c.w}, reinterpret_cast<u32x4 *>(dst));
}

// Fast-path epilogue of 16 consecutive accumulators of one row (per-tensor
// scales or raw INT32 output, column a multiple of 16, output and bias rows
// 16-byte aligned, all 16 inside the output): v = acc * sa * sb (+ bias),
// then one to four 16-byte stores; INT32 output stores the accumulators.
// Returns the running max |v| as FP32 bits.
// OD: the output dtype, fixed at compile time by the caller's dispatch;
// HB: whether a bias is present (its kind is still tested at run time).
// STAGE (BF16 output): the two 16-byte halves go to the LDS addresses
// stage0 / stage1 instead of the output, for a caller that writes whole
// lines.
template <bool INT_ACC, int OD, bool HB, bool STAGE = false>
__device__ __forceinline__ uint32_t nt_store16(const GemmParams &p, const Epilogue &epi, const uint4 (&w)[4],
                                               int64_t row, int64_t col, uint32_t vmax, float &macc,
                                               uint8_t *stage0 = nullptr, uint8_t *stage1 = nullptr)
{
    static_assert(!STAGE || OD == DT_BF16, "staged halves are BF16 rows");
    if constexpr (OD == DT_E4M3 && !HB) {
        *reinterpret_cast<uint4 *>(static_cast<uint8_t *>(p.out) + row * p.ldo + col) =
            nt_e4m3_codes16<INT_ACC>(epi, w, macc);
        return vmax;
    }
    if constexpr (INT_ACC && OD == DT_INT32) {
        uint4 *out = reinterpret_cast<uint4 *>(static_cast<int32_t *>(p.out) + row * p.ldo + col);
#pragma unroll
        for (int q = 0; q < 4; ++q) out[q] = w[q];
        return vmax;
    }
    auto val = [](uint32_t x) { return INT_ACC ? (float)(int32_t)x : __uint_as_float(x); };
    float v[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        v[4 * q + 0] = val(w[q].x) * epi.s_ab;
        v[4 * q + 1] = val(w[q].y) * epi.s_ab;
        v[4 * q + 2] = val(w[q].z) * epi.s_ab;
        v[4 * q + 3] = val(w[q].w) * epi.s_ab;
    }
    if constexpr (!HB) {
    } else if (p.bias_dt == DT_FP32) {
        const float4 *b = reinterpret_cast<const float4 *>(static_cast<const float *>(p.bias) + col);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 x = b[q];
            v[4 * q] += x.x; v[4 * q + 1] += x.y; v[4 * q + 2] += x.z; v[4 * q + 3] += x.w;
        }
    } else if (p.bias_dt == DT_BF16) {
        const uint4 *b = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(p.bias) + col);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const uint4 x = b[q];
            const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[8 * q + 2 * e] += bf16_lo(xs[e]);
                v[8 * q + 2 * e + 1] += bf16_hi(xs[e]);
            }
        }
    } else if (p.bias_dt == BIAS_Q_E4M3 || p.bias_dt == BIAS_Q_E5M2) {
        const uint4 x = *reinterpret_cast<const uint4 *>(static_cast<const uint8_t *>(p.bias) + col);
        const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
        const float bs = p.bias_scale[0];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const uint32_t c = (xs[e >> 2] >> (8 * (e & 3))) & 0xFFu;
            v[e] += (p.bias_dt == BIAS_Q_E4M3 ? fp8_decode<FMT_E4M3>(c) : fp8_decode<FMT_E5M2>(c)) * bs;
        }
    }
    {
        // max |v| as a float maximum with |.| source modifiers (three
        // operands per instruction); for the finite values of the contract
        // it is the maximum of the |v| bit patterns.
        float m = __builtin_fabsf(v[0]);
#pragma unroll
        for (int e = 1; e < 16; e += 2)
            m = __builtin_elementwise_maximum(
                m, __builtin_elementwise_maximum(__builtin_fabsf(v[e]), e + 1 < 16 ? __builtin_fabsf(v[e + 1]) : 0.0f));
        const uint32_t b = __float_as_uint(m);
        vmax = b > vmax ? b : vmax;
    }
    const int64_t o = row * p.ldo + col;
    if constexpr (OD == DT_E4M3) {
        const float s = epi.inv_os;
        uint4 c;
        c.x = encode4<FMT_E4M3>(v[0] * s, v[1] * s, v[2] * s, v[3] * s);
        c.y = encode4<FMT_E4M3>(v[4] * s, v[5] * s, v[6] * s, v[7] * s);
        c.z = encode4<FMT_E4M3>(v[8] * s, v[9] * s, v[10] * s, v[11] * s);
        c.w = encode4<FMT_E4M3>(v[12] * s, v[13] * s, v[14] * s, v[15] * s);
        *reinterpret_cast<uint4 *>(static_cast<uint8_t *>(p.out) + o) = c;
    } else if constexpr (OD == DT_BF16) {
        uint32_t hw[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            hw[e] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[2 * e]) |
                    ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[2 * e + 1]) << 16);
        if constexpr (STAGE) {
            *reinterpret_cast<uint4 *>(stage0) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
            *reinterpret_cast<uint4 *>(stage1) = make_uint4(hw[4], hw[5], hw[6], hw[7]);
        } else {
            uint4 *out = reinterpret_cast<uint4 *>(static_cast<uint16_t *>(p.out) + o);
            out[0] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
            out[1] = make_uint4(hw[4], hw[5], hw[6], hw[7]);
        }
    } else {
        float4 *out = reinterpret_cast<float4 *>(static_cast<float *>(p.out) + o);
#pragma unroll
        for (int q = 0; q < 4; ++q) out[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
    }
    return vmax;
}

template <int AF, int BF, bool KTAIL, bool CHAIN>
__global__ __launch_bounds__(GEMM_THREADS, 1) void qgemm_nt_kernel(GemmParams p)
{
    static_assert(!(CHAIN && KTAIL), "a chained grid needs whole k-steps");
    typedef Mma32<BF, AF> MMA;                 // operands swapped: acc holds C^T
    constexpr int RPS = NT_READS_PER_SLOT;
    typedef typename MMA::acc_t acc_t;
    constexpr int WM = NT_BM / 2, WN = NT_BN / 2, TM = WM / 32, TN = WN / 32;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[NT_STAGES * NT_STAGE_BYTES];
    __shared__ uint32_t red[GEMM_THREADS / 64];
    // E4M3 register epilogue: each wave turns a row of blocks (32 rows x
    // 128 bytes of codes) into whole 128-byte lines here.
    __shared__ __attribute__((aligned(16))) uint8_t ep_lines[(GEMM_THREADS / 64) * 32 * 128];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar LDS windows
    const int wm0 = (wave >> 1) * WM, wn0 = (wave & 1) * WN;
    const int total = p.tiles_m * p.tiles_n;

    // A tile's operand panels start at its first rows; rows past the
    // matrix are outside num_records and load as zeros.  The loop carries
    // base and size as plain scalars and each step builds the buffer
    // resources from them (a resource carried through the loop would be
    // treated as divergent).
    auto panel_bytes = [&](int64_t ld, int64_t rows_left) { return (int)(rows_left > 0 ? rows_left * ld : 0); };

    // LDS layout: [A stage 0 | A stage 1 | B stage 0 | B stage 1], 32 KiB
    // each, so a fragment read's stage and fragment offsets fit the
    // instruction's 16-bit immediate offset.
    //
    // Load j of this wave covers bytes [(jj*4 + wave) * 1024, +1024) of the
    // A part of a stage (j < NT_LOADS/2, jj = j) or of the B part (jj = j -
    // NT_LOADS/2).  Lane i lands at position q = (jj*4 + wave)*64 + i
    // (16-byte units): row q/8, swizzled chunk q%8, so it fetches logical
    // chunk (q%8) ^ f(row).  The step's k offset travels in the scalar
    // offset field, so a full step costs no vector instruction per load.
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
    const int nk = (int)((p.K + NT_BK - 1) / NT_BK);
    __builtin_assume(nk > 0);   // K == 0 never reaches this kernel
    const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_ptr_t)lds;
    const uint32_t lds_wave = lds_base + (uint32_t)wave * 1024u;   // wave-uniform: lands in M0
    // Direct-to-LDS load j (0 .. NT_LOADS-1) of the step at k offset k0 of
    // the panels (ra, rb) into stage S.  Without a K tail every step is
    // whole and k0 rides in the scalar offset.  With one (KTAIL), chunks at
    // or past K get an offset outside the buffer range and load as zeros,
    // which also covers the refills past the last step.
    auto issue_one = [&](auto S, int k0, int j, const __amdgpu_buffer_rsrc_t &ra, const __amdgpu_buffer_rsrc_t &rb) {
        constexpr int STAGE = decltype(S)::value;
        const bool is_a = j < NT_LOADS / 2;
        // The window base goes through an empty asm so each load adds its
        // constant in place (one scalar add) instead of the compiler keeping
        // 16 precomputed bases live, which the tile loop cannot afford.
        uint32_t wbase = lds_wave;
        asm volatile("" : "+s"(wbase));
        const lds_ptr_t dst = (lds_ptr_t)(uintptr_t)(wbase + (uint32_t)((is_a ? 0 : NT_STAGES * NT_A_BYTES) +
                                                                 STAGE * NT_A_BYTES + (j % (NT_LOADS / 2)) * 4096));
        if constexpr (!KTAIL) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(is_a ? ra : rb, dst, 16, (int)goff[j], k0, 0, 0);
        } else {
            const uint32_t off = k0 + kchunk[j] < K32 ? goff[j] + (uint32_t)k0 : BUF_OOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(is_a ? ra : rb, dst, 16, (int)off, 0, 0, 0);
        }
    };
    // k offset of the refill of `step`: steps past the end re-load the last
    // step (whole K) into a stage nobody reads, so the buffer offsets stay
    // inside the operands; with a K tail their chunks are all out of range.
    auto refill_k = [&](int step) { return (KTAIL || step < nk ? step : nk - 1) * NT_BK; };

    acc_t acc[TM][TN];

    const int lr = lane & 31, h = lane >> 5;
    // Per-lane read bases: a lane reads rows (wm0 | wn0) + f*32 + lr, and
    // only chunks 4*half + 2*h + e (half, e in {0, 1}).  The swizzle
    // depends on lr alone (f*32 and the wave offsets are multiples of 32),
    // so fragment f, stage s adds the immediate s*NT_A_BYTES + f*32*NT_BK.
    uint32_t rba[2][2], rbb[2][2];
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const uint32_t in_row = (uint32_t)(lr * NT_BK + (((4 * half + 2 * h + e) ^ nt_swz(lr)) << 4));
            rba[half][e] = lds_base + (uint32_t)(wm0 * NT_BK) + in_row;
            rbb[half][e] = lds_base + (uint32_t)(NT_STAGES * NT_A_BYTES + wn0 * NT_BK) + in_row;
        }
    // Fragment read t (0..15) of one 64-deep half: t/2 selects A fragment
    // 0..3 or B fragment 0..3, t%2 the 16-byte half.
    auto read_frag = [&](auto S, auto HALF, auto T) -> u32x4 {
        constexpr int STAGE = decltype(S)::value, HF = decltype(HALF)::value, t = decltype(T)::value;
        constexpr int f = t >> 1, e = t & 1;
        constexpr int off = STAGE * NT_A_BYTES + (f < TM ? f : f - TM) * 32 * NT_BK;
        return nt_read16<off>(f < TM ? rba[HF][e] : rbb[HF][e]);
    };
    typedef std::integral_constant<int, 0> I0;
    typedef std::integral_constant<int, 1> I1;
    constexpr int VM_ONE_STEP = 0x0F70 | (NT_LOADS & 0xF) | ((NT_LOADS >> 4) << 14);
    // Two fragment sets of 16 halves each: parts 2i, 2i+1 are A fragment i,
    // parts 2(TM+j), 2(TM+j)+1 B fragment j.
    u32x4 f0[16], f1[16];
    auto mma = [&](u32x4 (&f)[16], int t) {
        const int i = t >> 2, j = t & 3;
        MMA::run(acc[i][j], f[2 * (TM + j)], f[2 * (TM + j) + 1], f[2 * i], f[2 * i + 1]);
    };
    auto mma0 = [&](u32x4 (&f)[16], int t) {
        const int i = t >> 2, j = t & 3;
        MMA::run0(acc[i][j], f[2 * (TM + j)], f[2 * (TM + j) + 1], f[2 * i], f[2 * i + 1]);
    };

    // CHAIN (the launcher guarantees: every tile whole, the register
    // epilogue, an even number of whole k-steps): the next tile's first two
    // steps are fetched by this tile's last refills, since the epilogue
    // leaves the LDS stages alone and the next tile starts on stage 0.
    uint32_t vmax = 0;
    bool started = false;   // this tile's steps 0 and 1 are in flight and f0 holds its first fragments
    // The panels refills load from (this tile's, then the next one's).
    const uint8_t *pa = p.a, *pb = p.b;
    int na = 0, nb = 0;

    // The epilogue's scalars (product scale, output scale) are read once,
    // before any operand load is in flight: read inside the tile loop,
    // their wait would also wait for the next tile's first loads.
    const GemmParams &pe = p;
    const Epilogue epi(pe);

    // Without CHAIN the body runs once (one tile per workgroup).
    int id = (int)blockIdx.x;
    do {
        int tm, tn;
        tile_coords_of(id, p.tiles_m, p.tiles_n, tm, tn);
        const int64_t m0 = (int64_t)tm * NT_BM, n0 = (int64_t)tn * NT_BN;
        const bool whole = CHAIN || (m0 + NT_BM <= p.M && n0 + NT_BN <= p.N);
        const int next = id + (int)gridDim.x;
        const bool chain = CHAIN && next < total;


        // One k-step worked from stage S (= kt % 2).  Half 0: MFMAs on set 0
        // while half 1's fragments are read into set 1 (front-loaded,
        // NT_READS_PER_SLOT per MFMA slot); once every wave has them (the
        // barrier at slot NT_LOAD_SLOT0) stage S is refilled with step kt+2
        // -- of the next tile when chaining past the end -- one load per
        // slot (bursts overflow the texture address queue and stall the
        // wave).  At the mid-step barrier everyone's loads of step kt+1 have
        // landed.  Half 1: MFMAs on set 1 while step kt+1's half-0 fragments
        // are read from the other stage into set 0, and the refill goes on.
        auto step = [&](auto S, auto FIRST, int kt) {
            constexpr int STAGE = decltype(S)::value;
            typedef std::integral_constant<int, 1 - STAGE> SN;
            const bool to_next = chain && kt + 2 >= nk;
            if (chain && kt + 2 == nk) {
                int tm2, tn2;
                tile_coords_of(next, p.tiles_m, p.tiles_n, tm2, tn2);
                const int64_t m2 = (int64_t)tm2 * NT_BM, n2 = (int64_t)tn2 * NT_BN;
                pa = p.a + m2 * p.lda; na = panel_bytes(p.lda, p.M - m2);
                pb = p.b + n2 * p.ldb; nb = panel_bytes(p.ldb, p.N - n2);
            }
            const __amdgpu_buffer_rsrc_t la = __builtin_amdgcn_make_buffer_rsrc((void *)pa, (short)0, na, BUF_WORD3);
            const __amdgpu_buffer_rsrc_t lb = __builtin_amdgcn_make_buffer_rsrc((void *)pb, (short)0, nb, BUF_WORD3);
            const int k_refill = to_next ? (kt + 2 - nk) * NT_BK : refill_k(kt + 2);
            // Refill loads issued in slot t of half H (NT_LOAD_SLOT0 counts
            // slots across both halves).
            auto refills = [&](auto H, auto T) {
                constexpr int g = decltype(H)::value * 16 + decltype(T)::value - NT_LOAD_SLOT0;
                if constexpr (g >= 0)
                    nt_unroll<0, NT_LOADS_PER_SLOT>([&](auto U) {
                        constexpr int i = g * NT_LOADS_PER_SLOT + decltype(U)::value;
                        if constexpr (i < NT_LOADS) issue_one(S, k_refill, i, la, lb);
                    });
            };
            nt_unroll<0, 16>([&](auto T) {
                constexpr int t = decltype(T)::value;
                if constexpr (decltype(FIRST)::value) mma0(f0, t);
                else mma(f0, t);
                nt_unroll<0, RPS>([&](auto R) {
                    constexpr int r = t * RPS + decltype(R)::value;
                    if constexpr (r < 16) f1[r] = read_frag(S, I1{}, std::integral_constant<int, r>{});
                });
                if constexpr (NT_LOAD_SLOT0 < 16 && t == NT_LOAD_SLOT0) {
                    // Every wave has its fragments of stage S: it may refill.
                    nt_wait_parts(f1);
                    __builtin_amdgcn_s_barrier();
                }
                refills(I0{}, T);
                __builtin_amdgcn_sched_barrier(0);
            });
            // This wave's loads of step kt+1 have landed (all but the refill
            // loads issued since); after the barrier, everyone's have.
            nt_wait_parts(f1);
            __builtin_amdgcn_s_waitcnt(NT_VM_MID);
            __builtin_amdgcn_s_barrier();
            nt_unroll<0, 16>([&](auto T) {
                constexpr int t = decltype(T)::value;
                mma(f1, t);
                nt_unroll<0, RPS>([&](auto R) {
                    constexpr int r = t * RPS + decltype(R)::value;
                    if constexpr (r < 16) f0[r] = read_frag(SN{}, I0{}, std::integral_constant<int, r>{});
                });
                refills(I1{}, T);
                __builtin_amdgcn_sched_barrier(0);
            });
            nt_wait_parts(f0);
        };

        if (!started) {
            pa = p.a + m0 * p.lda; na = panel_bytes(p.lda, p.M - m0);
            pb = p.b + n0 * p.ldb; nb = panel_bytes(p.ldb, p.N - n0);
            const __amdgpu_buffer_rsrc_t la = __builtin_amdgcn_make_buffer_rsrc((void *)pa, (short)0, na, BUF_WORD3);
            const __amdgpu_buffer_rsrc_t lb = __builtin_amdgcn_make_buffer_rsrc((void *)pb, (short)0, nb, BUF_WORD3);
            __syncthreads();   // the previous tile's LDS epilogue is done with the stages
#pragma unroll
            for (int j = 0; j < NT_LOADS; ++j) issue_one(I0{}, 0, j, la, lb);
            if (nk > 1) {
#pragma unroll
                for (int j = 0; j < NT_LOADS; ++j) issue_one(I1{}, NT_BK, j, la, lb);
                __builtin_amdgcn_s_waitcnt(VM_ONE_STEP);
            } else {
                __builtin_amdgcn_s_waitcnt(0x0F70);
            }
            __builtin_amdgcn_s_barrier();
            nt_unroll<0, 16>([&](auto T) { f0[decltype(T)::value] = read_frag(I0{}, I0{}, T); });
            nt_wait_parts(f0);
        }
        // Steps past the end read stale fragments that no MFMA uses (or,
        // chaining, the next tile's first ones); the loop runs two steps per
        // iteration so each step's stage is a constant.  The first step's
        // first half starts every block from a zero accumulator (clearing
        // the 256 accumulator registers between two chained tiles cost
        // about 1%).
        step(I0{}, std::true_type{}, 0);
        if (1 < nk) step(I1{}, std::false_type{}, 1);
        for (int kt = 2; kt < nk; kt += 2) {
            step(I0{}, std::false_type{}, kt);
            if (kt + 1 < nk) step(I1{}, std::false_type{}, kt + 1);
        }
        if (!chain) {
            __builtin_amdgcn_s_waitcnt(0x0F70);
            __syncthreads();
        }
        started = chain;

        // Epilogue.  Block (i, j) holds C^T: element r of lane l is output row
        // i*32 + l%32, column j*32 + (r/4)*8 + 4*(l/32) + r%4.
        //
        // Fast path (whole tile inside the output, per-tensor scales, 16-byte
        // aligned output and bias rows): straight from registers.  Swapping the
        // upper half-wave of register quads 0 and 1 with the lower half-wave of
        // quads 2 and 3 (v_permlane32_swap) leaves lane l with the 16
        // consecutive columns 16*(l/32) .. +15 of its row, in quad order
        // 0, 2, 1, 3, which then go out as 16-byte stores.
        //
        // Otherwise through LDS, one 32-row slab of the wave tile at a time:
        // register quad q goes to LDS as one 16-byte write, then each lane takes
        // 4 columns at a time through the general epilogue with its bounds
        // checks.  With row stride EP_LD = 132 words, the 16 lanes that share an
        // LDS clock touch 16 distinct bank slots.
        // The register path, one row of blocks per iteration at run time,
        // its 4 blocks unrolled (keeps the code and register pressure
        // small); each block's accumulators are picked out through
        // compile-time indices.  The output dtype and the presence of a
        // bias are fixed per tile, so the blocks carry no tests for them.
        auto regs_rows = [&](auto OD_, auto HB_) {
            constexpr int OD = decltype(OD_)::value;
            constexpr bool HB = decltype(HB_)::value;
            float macc = 0.0f;   // max |acc| (E4M3 output without bias)
            uint8_t *const ep_wave = ep_lines + wave * 32 * 128;
#pragma unroll 1
            for (int i = 0; i < TM; ++i) {
                nt_unroll<0, TN>([&](auto J) {
                    constexpr int j = decltype(J)::value;
                    uint32_t x[16];
                    nt_unroll<0, TM>([&](auto I) {
                        constexpr int ii = decltype(I)::value;
                        if (i == ii) {
#pragma unroll
                            for (int r = 0; r < 16; ++r) x[r] = MMA::bits(acc[ii][j], r);
                        }
                    });
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const auto s02 = __builtin_amdgcn_permlane32_swap(x[r], x[8 + r], false, false);
                        x[r] = s02[0]; x[8 + r] = s02[1];
                        const auto s13 = __builtin_amdgcn_permlane32_swap(x[4 + r], x[12 + r], false, false);
                        x[4 + r] = s13[0]; x[12 + r] = s13[1];
                    }
                    const uint4 w[4] = {make_uint4(x[0], x[1], x[2], x[3]), make_uint4(x[8], x[9], x[10], x[11]),
                                        make_uint4(x[4], x[5], x[6], x[7]), make_uint4(x[12], x[13], x[14], x[15])};
                    if constexpr (OD == DT_E4M3 && !HB) {
                        // Codes of columns 32j + 16h .. +15 of row lr into
                        // the wave's staging lines.
                        const int c = 2 * j + h;
                        *reinterpret_cast<uint4 *>(ep_wave + lr * 128 + ((c ^ nt_line_swz(lr)) << 4)) =
                            nt_e4m3_codes16<MMA::INT_ACC>(epi, w, macc);
                    } else if constexpr (MMA::INT_ACC && OD == DT_INT32) {
                        // Raw INT32: the block's 32 rows x 128 bytes go
                        // through the staging lines on their own (lane:
                        // row lr, chunks 4h .. 4h+3), then out as whole
                        // lines, streamed like the E4M3 codes.
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            *reinterpret_cast<uint4 *>(ep_wave + lr * 128 + (((4 * h + q) ^ nt_line_swz(lr)) << 4)) = w[q];
                        const int ch = lane & 7;
                        nt_unroll<0, 4>([&](auto KK) {
                            constexpr int k = decltype(KK)::value;
                            const int r = 8 * k + (lane >> 3);
                            const uint4 v =
                                *reinterpret_cast<const uint4 *>(ep_wave + r * 128 + ((ch ^ nt_line_swz(r)) << 4));
                            nt_store16_stream(reinterpret_cast<uint8_t *>(static_cast<int32_t *>(pe.out) +
                                                                          (m0 + wm0 + i * 32 + r) * pe.ldo + n0 + wn0 +
                                                                          j * 32 + ch * 4),
                                              v);
                        });
                    } else {
                        const int64_t row = m0 + wm0 + i * 32 + lr;
                        const int64_t col = n0 + wn0 + j * 32 + h * 16;
                        vmax = nt_store16<MMA::INT_ACC, OD, HB>(pe, epi, w, row, col, vmax, macc);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                });
                if constexpr (OD == DT_E4M3 && !HB) {
                    // Whole lines out: store k covers rows 8k .. 8k+7 of the
                    // row of blocks, eight lanes (128 bytes) per row,
                    // streamed past the caches (a 128-byte line per eight
                    // lanes writes whole lines; the codes are not re-read
                    // by this kernel, and the memory-side cache stays with
                    // the operands).
                    const int ch = lane & 7;
                    nt_unroll<0, 4>([&](auto KK) {
                        constexpr int k = decltype(KK)::value;
                        const int r = 8 * k + (lane >> 3);
                        const uint4 v = *reinterpret_cast<const uint4 *>(ep_wave + r * 128 + ((ch ^ nt_line_swz(r)) << 4));
                        nt_store16_stream(static_cast<uint8_t *>(pe.out) + (m0 + wm0 + i * 32 + r) * pe.ldo + n0 + wn0 +
                                              ch * 16,
                                          v);
                    });
                }
            }
            if constexpr (OD == DT_E4M3 && !HB) {
                const uint32_t b = __float_as_uint(macc * __builtin_fabsf(epi.s_ab));
                vmax = b > vmax ? b : vmax;
            }
        };
        typedef std::integral_constant<bool, true> HasBias;
        typedef std::integral_constant<bool, false> NoBias;
        if (CHAIN || ((epi.per_tensor || p.out_dt == DT_INT32) && p.out_vec16 && p.bias_vec16 && whole)) {
            const bool hb = pe.bias_dt >= 0;
            if (MMA::INT_ACC && pe.out_dt == DT_INT32) {
                if constexpr (MMA::INT_ACC) regs_rows(std::integral_constant<int, DT_INT32>{}, NoBias{});
            } else if (pe.out_dt == DT_E4M3) {
                if (hb) regs_rows(std::integral_constant<int, DT_E4M3>{}, HasBias{});
                else regs_rows(std::integral_constant<int, DT_E4M3>{}, NoBias{});
            } else if (pe.out_dt == DT_BF16) {
                if (hb) regs_rows(std::integral_constant<int, DT_BF16>{}, HasBias{});
                else regs_rows(std::integral_constant<int, DT_BF16>{}, NoBias{});
            } else {
                if (hb) regs_rows(std::integral_constant<int, DT_FP32>{}, HasBias{});
                else regs_rows(std::integral_constant<int, DT_FP32>{}, NoBias{});
            }
        } else if constexpr (!CHAIN) {
            constexpr int EP_LD = WN + 4;                    // padded row, in words
            uint32_t *ep = reinterpret_cast<uint32_t *>(lds) + wave * 32 * EP_LD;
            // The slab loop runs at run time (its body is large); the accumulator
            // rows go to LDS through compile-time indices so they stay in
            // registers.
#pragma unroll 1
            for (int i = 0; i < TM; ++i) {
                __syncthreads();
                nt_unroll<0, TM>([&](auto I) {
                    constexpr int ii = decltype(I)::value;
                    if (i == ii) {
#pragma unroll
                        for (int j = 0; j < TN; ++j)
#pragma unroll
                            for (int q = 0; q < 4; ++q)
                                *reinterpret_cast<uint4 *>(ep + lr * EP_LD + j * 32 + q * 8 + h * 4) =
                                    make_uint4(MMA::bits(acc[ii][j], 4 * q), MMA::bits(acc[ii][j], 4 * q + 1),
                                               MMA::bits(acc[ii][j], 4 * q + 2), MMA::bits(acc[ii][j], 4 * q + 3));
                    }
                });
                __syncthreads();
                constexpr int C4 = WN / 4, PER_LANE = 32 * C4 / 64, GROUP = 8;
#pragma unroll 1
                for (int g = 0; g < PER_LANE; g += GROUP) {
                    uint4 w[GROUP];
#pragma unroll
                    for (int u = 0; u < GROUP; ++u) {
                        const int idx = lane + (g + u) * 64;
                        w[u] = *reinterpret_cast<const uint4 *>(ep + (idx / C4) * EP_LD + (idx % C4) * 4);
                    }
#pragma unroll
                    for (int u = 0; u < GROUP; ++u) {
                        const int idx = lane + (g + u) * 64;
                        const int64_t row = m0 + wm0 + i * 32 + idx / C4;
                        const int64_t col = n0 + wn0 + (idx % C4) * 4;
                        if (row < pe.M && col < pe.N) vmax = epi.store4<MMA::INT_ACC>(w[u], row, col, vmax);
                    }
                }
            }
        }
        if constexpr (!CHAIN) break;
        id = next;
    } while (id < total);
    if (p.out_amax) gemm_publish_amax(p, vmax, red);
}

template <int AF, int BF>
hipError_t launch_nt(GemmParams p, hipStream_t s)
{
    p.tiles_m = (int)((p.M + NT_BM - 1) / NT_BM);
    p.tiles_n = (int)((p.N + NT_BN - 1) / NT_BN);
    // Chained (persistent: one workgroup per CU -- its LDS and registers
    // allow no more -- each walking every grid-th tile) when every tile is
    // whole, takes the register epilogue, and K is an even number of whole
    // steps; otherwise one tile per workgroup.
    const int64_t tiles = (int64_t)p.tiles_m * p.tiles_n;
    const int64_t cus = device_cu_count();
    const bool chain = p.M % NT_BM == 0 && p.N % NT_BN == 0 && p.K % (2 * NT_BK) == 0 &&
                       ((p.sa_group == 0 && p.sb_group == 0) || p.out_dt == DT_INT32) && p.out_vec16 &&
                       p.bias_vec16 && tiles > cus;
    const int64_t grid = chain ? cus : tiles;
    p.amax_part = gemm_amax_parts(p.amax_part, grid);
    if (chain)
        hipLaunchKernelGGL((qgemm_nt_kernel<AF, BF, false, true>), dim3((unsigned)grid), dim3(GEMM_THREADS), 0, s, p);
    else if (p.K % NT_BK == 0)
        hipLaunchKernelGGL((qgemm_nt_kernel<AF, BF, false, false>), dim3((unsigned)grid), dim3(GEMM_THREADS), 0, s, p);
    else
        hipLaunchKernelGGL((qgemm_nt_kernel<AF, BF, true, false>), dim3((unsigned)grid), dim3(GEMM_THREADS), 0, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || !p.out_amax || !p.amax_part) return e;
    return launch_amax_finalize(p, grid, s);
}

}  // namespace ql
