// qgemm_pipe.hpp -- pipelined scaled GEMM for products with few output
// tiles (the MLP-up forward and the backward's dX / dW shapes of AstrAI
// ops/fp8.py @5e76fbd: linear_forward_fp8, linear_backward_fp8), gfx950.
//
//   out[m, n] = (sum_k A[m, k] * B[n, k]) * sa * sb (+ bias[n])
//
// The schedule of the large K-major kernel (qgemm_nt.hpp), for BM x BN
// tiles smaller than 256 x 256 (so that a product with a few thousand rows
// still gives every CU a tile) and for either operand stored MN-major:
//   * 4 waves, 2 x 2, each owning (BM/2) x (BN/2) as 32 x 32 blocks of
//     v_mfma_f32_32x32x64_f8f6f4 (INT8: two v_mfma_i32_32x32x32_i8), the
//     operands swapped so each lane's accumulator quad holds 4 consecutive
//     output columns.
//   * K in steps of 128 bytes through a ring of 3 or 4 LDS stages, filled
//     global -> LDS by buffer loads with an LDS destination (no registers):
//     step k refills its stage with step k + STAGES.  A step is two
//     64-deep halves with two fragment register sets: half 0's matrix ops
//     run while half 1's fragments are read; once every wave has them (a
//     barrier) the stage is refilled with step k + STAGES, spread over
//     the step's remaining matrix-op slots; after the mid-step wait and
//     barrier, half 1's matrix ops run while the next step's first
//     fragments are read.
//   * A K-major operand: rows of 128 k-bytes, 16-byte chunk c of row r at
//     position c ^ ((r >> 1) & 7), read with ds_read_b128 (two per 32 x 64
//     fragment).
//   * An MN-major operand: stored as it lies in memory, one k-row of R
//     mn-bytes (R = tile rows) per k, chunk c of k-row kr at position
//     c ^ s(kr), read with ds_read_b64_tr_b8 (four per fragment): within a
//     16-lane block, lanes 2j and 2j+1 address k-row k0 + j at mn bytes
//     [m, m + 8) and [m + 8, m + 16), and lane i receives k0 .. k0 + 7 of mn
//     row m + i.  Lane l (block b = l >> 4, t = l & 15) of a fragment reads
//     k-rows 64*half + 32*(b >> 1) + 8*q + (t >> 1), q = 0..3, at chunk
//     (row0 + 16*(b & 1)) / 16: 16 consecutive rows per block, 32
//     consecutive k per lane, the K-major fragment's lane layout.
//     s(kr) = 2*((kr >> log2(256/R)) & (R/32 - 1)) | ((kr >> 5) & 1) puts
//     the 16 (k-row, chunk) pairs that any 32 lanes of one read touch (8
//     k-rows x 2 chunks, or the same at k-rows 32 apart) on distinct banks
//     (brute-force checked).
// Requirements (host side, p.fast): 16-byte aligned operands and leading
// dimensions, K % 16 == 0 for a K-major and MN % 16 == 0 for an MN-major
// operand, byte offsets below 2^31.  Rows past M / N of a K-major operand
// and k-rows past K of an MN-major one are outside the buffer range and read
// as zeros; K-major chunks past K are sent outside it.  An MN-major tile may
// read bytes of columns past M (N) inside the buffer; they only reach
// accumulator rows that are never stored.
#pragma once

#include "qgemm_nt.hpp"

namespace ql {

template <int R> __device__ __forceinline__ int pipe_mn_swz(int kr)
{
    static_assert(R == 256 || R == 128 || R == 64, "MN-major tile rows");
    constexpr int SH = R == 256 ? 0 : (R == 128 ? 1 : 2);
    constexpr int MSK = R / 32 - 1;
    return (((kr >> SH) & MSK) << 1) | ((kr >> 5) & 1);
}

template <int OFF>
__device__ __forceinline__ u32x2 pipe_read_tr8(uint32_t addr)
{
    static_assert(OFF >= 0 && OFF < 65536, "LDS immediate offset is 16 bits");
    u32x2 x;
    asm volatile("ds_read_b64_tr_b8 %0, %1 offset:%2" : "=v"(x) : "v"(addr), "n"(OFF) : "memory");
    return x;
}

// A fragment in registers: 32 bytes per lane as two 16-byte reads
// (K-major) or four 8-byte transpose reads (MN-major).
template <bool MN> struct PipeFrag;
template <> struct PipeFrag<false> {
    static constexpr int READS = 2;
    u32x4 h[2];
    __device__ __forceinline__ void tie() { asm volatile("" : "+v"(h[0]), "+v"(h[1])); }
    __device__ __forceinline__ u32x4 lo() const { return h[0]; }
    __device__ __forceinline__ u32x4 hi() const { return h[1]; }
};
template <> struct PipeFrag<true> {
    static constexpr int READS = 4;
    u32x2 q[4];
    __device__ __forceinline__ void tie() { asm volatile("" : "+v"(q[0]), "+v"(q[1]), "+v"(q[2]), "+v"(q[3])); }
    __device__ __forceinline__ u32x4 lo() const { return u32x4{q[0].x, q[0].y, q[1].x, q[1].y}; }
    __device__ __forceinline__ u32x4 hi() const { return u32x4{q[2].x, q[2].y, q[3].x, q[3].y}; }
};

// One operand: R tile rows (BM for A, BN for B), PART = its LDS byte offset
// (stage s at PART + s * BYTES).  Loads: load j of wave w fills bytes
// [(4j + w) * 1024, +1024) of a stage's part, lane i at 16*i of that.
template <int R, bool MN, int PART> struct PipeOp {
    static constexpr int BYTES = R * 128;                          // one stage
    static constexpr int LOADS = BYTES / (GEMM_THREADS * 16);      // per thread per step
    static constexpr int T = R / 64;                               // fragments per wave (R/2 rows / 32)
    static constexpr int READS = PipeFrag<MN>::READS;              // per fragment per half
    const uint8_t *base;                                           // buffer base and size (resources built per load)
    int size;
    uint32_t goff[LOADS];
    int kc[LOADS];
    uint32_t ld32;
    // Read addresses (stage 0): K-major [half][e] (fragment f adds the
    // immediate f*32*128); MN-major [half][f*4 + q].
    uint32_t rd[2][MN ? T * 4 : 2];

    __device__ __forceinline__ void init(const uint8_t *ptr, int64_t ld, int64_t row0, int64_t rows_total,
                                         int64_t K, int wave, int lane, int wrow0, uint32_t lds_base)
    {
        ld32 = (uint32_t)ld;
        int64_t bytes;
        if constexpr (!MN) {
            const int64_t left = rows_total - row0;
            bytes = left > 0 ? left * ld : 0;
            base = ptr + row0 * ld;
        } else {
            bytes = row0 < rows_total ? K * ld - row0 : 0;
            base = ptr + row0;
        }
        size = (int)(bytes > 0 ? (bytes < 0x7FFFFFFF ? bytes : 0x7FFFFFFF) : 0);
#pragma unroll
        for (int j = 0; j < LOADS; ++j) {
            const int L = ((j * 4 + wave) * 64 + lane) * 16;         // byte within the stage's part
            if constexpr (!MN) {
                const int row = L >> 7;
                const int c = ((L >> 4) & 7) ^ nt_swz(row);
                kc[j] = c * 16;
                goff[j] = (uint32_t)(row * ld + c * 16);
            } else {
                const int kr = L / R;
                const int c = ((L % R) >> 4) ^ pipe_mn_swz<R>(kr);
                kc[j] = 0;
                goff[j] = (uint32_t)(kr * ld + c * 16);
            }
        }
        const int lr = lane & 31, h = lane >> 5;
        if constexpr (!MN) {
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int e = 0; e < 2; ++e)
                    rd[hf][e] = lds_base + PART + (uint32_t)((wrow0 + lr) * 128 + (((4 * hf + 2 * h + e) ^ nt_swz(lr)) << 4));
        } else {
            const int b = lane >> 4, t = lane & 15;
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int f = 0; f < T; ++f)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int kr = 64 * hf + 32 * (b >> 1) + 8 * q + (t >> 1);
                        const int c = (wrow0 + 32 * f + 16 * (b & 1)) >> 4;
                        rd[hf][f * 4 + q] = lds_base + PART +
                                            (uint32_t)(kr * R + ((c ^ pipe_mn_swz<R>(kr)) << 4) + 8 * (t & 1));
                    }
        }
        (void)h;
    }

    // Load j of the step at k offset k0 into stage S.
    template <int S, bool KTAIL>
    __device__ __forceinline__ void issue(int j, int k0, int K, uint32_t lds_wave) const
    {
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, size, BUF_WORD3);
        uint32_t wb = lds_wave;
        asm volatile("" : "+s"(wb));
        const lds_ptr_t dst = (lds_ptr_t)(uintptr_t)(wb + (uint32_t)(PART + S * BYTES + j * 4096));
        if constexpr (!MN) {
            if constexpr (!KTAIL) {
                __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, (int)goff[j], k0, 0, 0);
            } else {
                const uint32_t off = k0 + kc[j] < K ? goff[j] + (uint32_t)k0 : BUF_OOB;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, (int)off, 0, 0, 0);
            }
        } else {
            // The k offset rides in the vector offset, so k-rows past K are
            // outside the checked range (KTAIL or not).
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, (int)(goff[j] + (uint32_t)k0 * ld32), 0, 0, 0);
        }
    }

    // Read r (0 .. READS-1) of fragment f, half HF, stage S.
    template <int S, int HF, int F, int RR>
    __device__ __forceinline__ void read(PipeFrag<MN> &fr) const
    {
        // The stage and fragment offsets ride in the 16-bit immediate; past
        // 64 KiB the base takes 64 KiB of it.
        constexpr int OFF = S * BYTES + (MN ? 0 : F * 32 * 128);
        constexpr int IMM = OFF < 65536 ? OFF : OFF - 65536;
        const uint32_t a = MN ? rd[HF][F * 4 + RR] : rd[HF][RR];
        const uint32_t ab = OFF < 65536 ? a : a + 65536u;
        if constexpr (!MN) fr.h[RR] = nt_read16<IMM>(ab);
        else fr.q[RR] = pipe_read_tr8<IMM>(ab);
    }
};

// OCC workgroups per CU (their LDS stages must fit together), so the
// register allocator may use 1/OCC of the register file.
template <int AF, int BF, bool A_MN, bool B_MN, int BM, int BN, int STAGES, bool KTAIL, int OCC>
__global__ __launch_bounds__(GEMM_THREADS, OCC) __attribute__((amdgpu_waves_per_eu(OCC, OCC))) void qgemm_pipe_kernel(
    GemmParams p)
{
    typedef Mma32<BF, AF> MMA;                 // operands swapped: acc holds C^T
    typedef typename MMA::acc_t acc_t;
    constexpr int WM = BM / 2, WN = BN / 2, TM = WM / 32, TN = WN / 32;
    static_assert(STAGES >= 2 && STAGES <= 4, "LDS stages");
    constexpr int A_PART = 0, B_PART = STAGES * BM * 128;
    typedef PipeOp<BM, A_MN, A_PART> OpA;
    typedef PipeOp<BN, B_MN, B_PART> OpB;
    constexpr int LDS_BYTES = STAGES * (OpA::BYTES + OpB::BYTES);
    constexpr int LOADS = OpA::LOADS + OpB::LOADS;                 // per thread per step
    constexpr int RA = OpA::READS, RB = OpB::READS;
    constexpr int NR = TM * RA + TN * RB;                           // reads per half
    constexpr int SL = TM * TN;                                     // matrix-op slots per half
    // Fragment reads front-loaded RPS per slot; the refill starts two slots
    // after the last read of the half (at the latest in its last slot) and
    // goes LPS loads per slot over the rest of the step.
    constexpr int RPS = (NR + SL - 1) / SL > 2 ? (NR + SL - 1) / SL : 2;
    constexpr int R_END = (NR + RPS - 1) / RPS;
    constexpr int BAR = R_END + 2 < SL - 1 ? R_END + 2 : SL - 1;
    constexpr int LPS = (LOADS + (2 * SL - BAR) - 1) / (2 * SL - BAR);
    constexpr int EARLY = (SL - BAR) * LPS < LOADS ? (SL - BAR) * LPS : LOADS;   // refill loads in half 0
    // Loads that may stay in flight: at the mid-step wait of step kt, those
    // of steps kt+2 .. kt+STAGES-1 and this step's refills so far; at the
    // start, those of steps 1 .. STAGES-1.
    constexpr int MID = (STAGES - 2) * LOADS + EARLY, ONE = (STAGES - 1) * LOADS;
    static_assert(MID < 64 && (STAGES - 1) * LOADS < 64, "vmcnt holds 6 bits");
    constexpr int VM_MID = 0x0F70 | (MID & 0xF) | ((MID >> 4) << 14);
    constexpr int VM_ONE = 0x0F70 | (ONE & 0xF) | ((ONE >> 4) << 14);
    __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_BYTES];
    __shared__ uint32_t red[GEMM_THREADS / 64];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm0 = (wave >> 1) * WM, wn0 = (wave & 1) * WN;
    int tm, tn;
    tile_coords(p.tiles_m, p.tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_ptr_t)lds;
    const uint32_t lds_wave = lds_base + (uint32_t)wave * 1024u;

    OpA opa;
    OpB opb;
    opa.init(p.a, p.lda, m0, p.M, p.K, wave, lane, wm0, lds_base);
    opb.init(p.b, p.ldb, n0, p.N, p.K, wave, lane, wn0, lds_base);
    const int K32 = (int)p.K;
    const int nk = (int)((p.K + 127) / 128);
    __builtin_assume(nk > 0);
    // Refill of `step`: steps past the end re-load the last step (or, with
    // a K tail, chunks all out of range) into a stage nobody reads.
    auto refill_k = [&](int step) { return (KTAIL || step < nk ? step : nk - 1) * 128; };
    auto issue_load = [&](auto S, int i, int k0) {
        constexpr int ST = decltype(S)::value;
        if (i < OpA::LOADS) opa.template issue<ST, KTAIL>(i, k0, K32, lds_wave);
        else opb.template issue<ST, KTAIL>(i - OpA::LOADS, k0, K32, lds_wave);
    };

    acc_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = acc_t{};

    PipeFrag<A_MN> fa0[TM], fa1[TM];
    PipeFrag<B_MN> fb0[TN], fb1[TN];
    // Read t (0 .. NR-1) of a half: A fragments first, then B.
    auto read_t = [&](auto S, auto HF, auto T, PipeFrag<A_MN>(&fa)[TM], PipeFrag<B_MN>(&fb)[TN]) {
        constexpr int ST = decltype(S)::value, H = decltype(HF)::value, t = decltype(T)::value;
        if constexpr (t < TM * RA) opa.template read<ST, H, t / RA, t % RA>(fa[t / RA]);
        else opb.template read<ST, H, (t - TM * RA) / RB, (t - TM * RA) % RB>(fb[(t - TM * RA) / RB]);
    };
    auto wait_tie = [&](PipeFrag<A_MN>(&fa)[TM], PipeFrag<B_MN>(&fb)[TN]) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int i = 0; i < TM; ++i) fa[i].tie();
#pragma unroll
        for (int j = 0; j < TN; ++j) fb[j].tie();
    };
    auto mma = [&](PipeFrag<A_MN>(&fa)[TM], PipeFrag<B_MN>(&fb)[TN], int t) {
        const int i = t / TN, j = t % TN;
        MMA::run(acc[i][j], fb[j].lo(), fb[j].hi(), fa[i].lo(), fa[i].hi());
    };
    typedef std::integral_constant<int, 0> I0;
    typedef std::integral_constant<int, 1> I1;

    // One k-step from stage S (holding step kt; set 0 holds its half-0
    // fragments).
    auto step = [&](auto S, int kt) {
        constexpr int ST = decltype(S)::value;
        typedef std::integral_constant<int, (ST + 1) % STAGES> SN;
        const int k_refill = refill_k(kt + STAGES);
        auto refills = [&](auto H, auto T) {
            constexpr int g = decltype(H)::value * SL + decltype(T)::value - BAR;
            if constexpr (g >= 0)
                nt_unroll<0, LPS>([&](auto U) {
                    constexpr int i = g * LPS + decltype(U)::value;
                    if constexpr (i < LOADS) issue_load(S, i, k_refill);
                });
        };
        nt_unroll<0, SL>([&](auto T) {
            constexpr int t = decltype(T)::value;
            mma(fa0, fb0, t);
            nt_unroll<0, RPS>([&](auto R) {
                constexpr int r = t * RPS + decltype(R)::value;
                if constexpr (r < NR) read_t(S, I1{}, std::integral_constant<int, r>{}, fa1, fb1);
            });
            if constexpr (t == BAR) {
                // Every wave holds its fragments of stage S: it may refill.
                wait_tie(fa1, fb1);
                __builtin_amdgcn_s_barrier();
            }
            refills(I0{}, T);
            __builtin_amdgcn_sched_barrier(0);
        });
        // This wave's loads of step kt+1 have landed (all but the refill
        // loads issued since); after the barrier, everyone's have.
        wait_tie(fa1, fb1);
        __builtin_amdgcn_s_waitcnt(VM_MID);
        __builtin_amdgcn_s_barrier();
        nt_unroll<0, SL>([&](auto T) {
            constexpr int t = decltype(T)::value;
            mma(fa1, fb1, t);
            nt_unroll<0, RPS>([&](auto R) {
                constexpr int r = t * RPS + decltype(R)::value;
                if constexpr (r < NR) read_t(SN{}, I0{}, std::integral_constant<int, r>{}, fa0, fb0);
            });
            refills(I1{}, T);
            __builtin_amdgcn_sched_barrier(0);
        });
        wait_tie(fa0, fb0);
    };

    // Prologue: steps 0 .. STAGES-1 in flight (one per stage), step 0's
    // half-0 fragments read.
#pragma unroll
    for (int i = 0; i < LOADS; ++i) issue_load(I0{}, i, refill_k(0));
    nt_unroll<1, STAGES>([&](auto S) {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) issue_load(S, i, refill_k(decltype(S)::value));
    });
    __builtin_amdgcn_s_waitcnt(VM_ONE);
    __builtin_amdgcn_s_barrier();
    nt_unroll<0, NR>([&](auto T) { read_t(I0{}, I0{}, T, fa0, fb0); });
    wait_tie(fa0, fb0);
    // STAGES steps per iteration, so each step's stage is a constant.
    for (int kt = 0; kt < nk; kt += STAGES) {
        step(I0{}, kt);
        nt_unroll<1, STAGES>([&](auto S) {
            if (kt + decltype(S)::value < nk) step(S, kt + decltype(S)::value);
        });
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();

    // Epilogue.  Block (i, j) holds C^T: element r of lane l is output row
    // i*32 + l%32, column j*32 + (r/4)*8 + 4*(l/32) + r%4.
    const int lr = lane & 31, h = lane >> 5;
    const Epilogue epi(p);
    uint32_t vmax = 0;
    const bool whole = m0 + BM <= p.M && n0 + BN <= p.N;
    auto regs_rows = [&](auto OD_, auto HB_) {
        constexpr int OD = decltype(OD_)::value;
        constexpr bool HB = decltype(HB_)::value;
        // BF16 rows of a 64-column wave tile are 128 bytes: each row of
        // blocks goes through 4 KiB of LDS per wave (the stages are free
        // now) and out as whole lines.
        constexpr bool LINES = OD == DT_BF16 && WN == 64;
        uint8_t *const ep_wave = lds + wave * 32 * 128;
        float macc = 0.0f;
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
                const int64_t row = m0 + wm0 + i * 32 + lr;
                const int64_t col = n0 + wn0 + j * 32 + h * 16;
                if constexpr (LINES) {
                    // BF16 columns 32j + 16h .. +15 of row lr: chunks
                    // 4j + 2h and 4j + 2h + 1 of the row's 128 bytes.
                    const int c = 4 * j + 2 * h;
                    vmax = nt_store16<MMA::INT_ACC, OD, HB, true>(
                        p, epi, w, row, col, vmax, macc, ep_wave + lr * 128 + ((c ^ nt_line_swz(lr)) << 4),
                        ep_wave + lr * 128 + (((c + 1) ^ nt_line_swz(lr)) << 4));
                } else {
                    vmax = nt_store16<MMA::INT_ACC, OD, HB>(p, epi, w, row, col, vmax, macc);
                }
                __builtin_amdgcn_sched_barrier(0);
            });
            if constexpr (LINES) {
                // Whole 128-byte lines out, streamed past the caches: store
                // k covers rows 8k .. 8k+7 of the row of blocks, eight lanes
                // per row (MLP-up forward 15.7 -> 15.1 us, dW 12.9 -> 12.6
                // us; plain stores of the same lines: 15.3 and 13.0 us).
                const int ch = lane & 7;
                nt_unroll<0, 4>([&](auto KK) {
                    constexpr int k = decltype(KK)::value;
                    const int r = 8 * k + (lane >> 3);
                    const uint4 v = *reinterpret_cast<const uint4 *>(ep_wave + r * 128 + ((ch ^ nt_line_swz(r)) << 4));
                    nt_store16_stream(reinterpret_cast<uint8_t *>(static_cast<uint16_t *>(p.out) +
                                                                  (m0 + wm0 + i * 32 + r) * p.ldo + n0 + wn0 + ch * 8),
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
    if ((epi.per_tensor || p.out_dt == DT_INT32) && p.out_vec16 && p.bias_vec16 && whole) {
        const bool hb = p.bias_dt >= 0;
        if (MMA::INT_ACC && p.out_dt == DT_INT32) {
            if constexpr (MMA::INT_ACC) regs_rows(std::integral_constant<int, DT_INT32>{}, NoBias{});
        } else if (p.out_dt == DT_E4M3) {
            if (hb) regs_rows(std::integral_constant<int, DT_E4M3>{}, HasBias{});
            else regs_rows(std::integral_constant<int, DT_E4M3>{}, NoBias{});
        } else if (p.out_dt == DT_BF16) {
            if (hb) regs_rows(std::integral_constant<int, DT_BF16>{}, HasBias{});
            else regs_rows(std::integral_constant<int, DT_BF16>{}, NoBias{});
        } else {
            if (hb) regs_rows(std::integral_constant<int, DT_FP32>{}, HasBias{});
            else regs_rows(std::integral_constant<int, DT_FP32>{}, NoBias{});
        }
    } else {
        // Through LDS, one 32-row slab of the wave tile at a time (the
        // general epilogue with its bounds checks).
        constexpr int EP_LD = WN + 4;
        uint32_t *ep = reinterpret_cast<uint32_t *>(lds) + wave * 32 * EP_LD;
        static_assert(4 * 32 * EP_LD * 4 <= LDS_BYTES, "epilogue slab fits the stages");
        // The slab loop is unrolled (slab i picks its accumulators by a
        // compile-time index; a run-time one here, next to the register
        // path's, made the compiler reserve a stack frame).
        nt_unroll<0, TM>([&](auto I) {
            constexpr int i = decltype(I)::value;
            __syncthreads();
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    *reinterpret_cast<uint4 *>(ep + lr * EP_LD + j * 32 + q * 8 + h * 4) =
                        make_uint4(MMA::bits(acc[i][j], 4 * q), MMA::bits(acc[i][j], 4 * q + 1),
                                   MMA::bits(acc[i][j], 4 * q + 2), MMA::bits(acc[i][j], 4 * q + 3));
            __syncthreads();
            constexpr int C4 = WN / 4, PER_LANE = 32 * C4 / 64;
#pragma unroll 1
            for (int g = 0; g < PER_LANE; ++g) {
                const int idx = lane + g * 64;
                const uint4 w = *reinterpret_cast<const uint4 *>(ep + (idx / C4) * EP_LD + (idx % C4) * 4);
                const int64_t row = m0 + wm0 + i * 32 + idx / C4;
                const int64_t col = n0 + wn0 + (idx % C4) * 4;
                if (row < p.M && col < p.N) vmax = epi.store4<MMA::INT_ACC>(w, row, col, vmax);
            }
        });
    }
    if (p.out_amax) gemm_publish_amax(p, vmax, red);
}

// OCC = 1: one workgroup per CU with as many LDS stages as fit in 128 KiB
// (3 of 48 KiB for 256 x 128, 4 of 32 or 24 KiB for 128 x 128 and
// 128 x 64), so the loads of a step have that many steps to arrive.
// OCC = 2: two workgroups per CU with 2 stages each, so one workgroup's
// matrix ops run while the other waits (measured faster on the MLP-up
// forward, 2048 x 4096 x 1024 in 128 x 128 tiles, and slower on dW).
template <int AF, int BF, bool A_MN, bool B_MN, int BM, int BN, int OCC>
hipError_t launch_pipe(GemmParams p, hipStream_t s)
{
    constexpr int STAGES = OCC == 2 ? 2 : ((BM + BN) * 128 * 4 <= 128 * 1024 ? 4 : 3);
    static_assert(OCC * STAGES * (BM + BN) * 128 <= 160 * 1024, "LDS stages of the resident workgroups");
    p.tiles_m = (int)((p.M + BM - 1) / BM);
    p.tiles_n = (int)((p.N + BN - 1) / BN);
    const int64_t grid = (int64_t)p.tiles_m * p.tiles_n;
    p.amax_part = gemm_amax_parts(p.amax_part, grid);
    if (p.K % 128 == 0)
        hipLaunchKernelGGL((qgemm_pipe_kernel<AF, BF, A_MN, B_MN, BM, BN, STAGES, false, OCC>), dim3((unsigned)grid),
                           dim3(GEMM_THREADS), 0, s, p);
    else
        hipLaunchKernelGGL((qgemm_pipe_kernel<AF, BF, A_MN, B_MN, BM, BN, STAGES, true, OCC>), dim3((unsigned)grid),
                           dim3(GEMM_THREADS), 0, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || !p.out_amax || !p.amax_part) return e;
    return launch_amax_finalize(p, grid, s);
}

}  // namespace ql
