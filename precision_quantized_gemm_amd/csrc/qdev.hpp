// qdev.hpp -- device-side helpers shared by the quantize and GEMM kernels
// (gfx950 / CDNA4, wave64).
//
// Number formats: OCP E4M3 "fn" (largest finite 448) and E5M2 (57344), and
// symmetric INT8 in [-127, 127] -- the formats of AstrAI ops/fp8.py @5e76fbd
// (_fmt_dtype) and of the POPCORNBENCH "Kimi-K2.6 l2_p13" INT8 fake-quant
// (steps 2-4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ql {

enum : int { FMT_E4M3 = 0, FMT_E5M2 = 1, FMT_INT8 = 2 };
enum : int { DT_BF16 = 0, DT_FP32 = 1, DT_E4M3 = 2, DT_INT32 = 3 };

// Largest code magnitude (qmax in scale = amax / qmax) and amax floor.  The
// floors are the FP32 values nearest 1e-12 (FP8: the amax clamp of AstrAI's
// CPU quantize) and 1e-8 (INT8: the clamp of the POPCORNBENCH reference).
template <int FMT> struct Fmt;
template <> struct Fmt<FMT_E4M3> { static constexpr float qmax = 448.0f;   static constexpr float floor = 1e-12f; };
template <> struct Fmt<FMT_E5M2> { static constexpr float qmax = 57344.0f; static constexpr float floor = 1e-12f; };
template <> struct Fmt<FMT_INT8> { static constexpr float qmax = 127.0f;   static constexpr float floor = 1e-8f; };

// ---------------------------------------------------------------------------
// BF16 words: a 32-bit word holds two BF16 values, element 0 in the low half.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// |x| as FP32 bit patterns: non-negative floats order like their bits, so a
// maximum can be taken (and published with an atomic) on integers.
__device__ __forceinline__ uint32_t absbits_bf16_pair(uint32_t w)
{
    uint32_t lo = w & 0x7FFFu, hi = (w >> 16) & 0x7FFFu;
    return (lo > hi ? lo : hi) << 16;
}
__device__ __forceinline__ uint32_t absbits_f32(float x) { return __float_as_uint(x) & 0x7FFFFFFFu; }

// ---------------------------------------------------------------------------
// Correctly rounded x / s for a step s that is the same for many x.
//
// inv must be RN(1/s) (an IEEE division, done once).  Then q0 = RN(x*inv) is
// within one ulp of x/s, the residual r = x - q0*s is exact (one FMA), and
// RN(q0 + r*inv) is the correctly rounded quotient (Markstein, "Computation
// of elementary functions on the IBM RISC System/6000 processor", IBM J. Res.
// Dev. 1990).  The residual is exact as long as nothing underflows, which the
// caller guarantees by taking this path only for 2^-64 <= s <= 2^64: then a
// quotient large enough to matter for any code (>= 2^-17) implies
// |x| >= 2^-81.  Quotients far beyond every format's range (|q0| >= 2^120,
// including an overflow to inf) skip the correction; they saturate anyway.
// A zero q0 is returned as is: the correction would turn -0 into +0
// (-0 + +0 = +0 under round-to-nearest), and the sign of a zero quotient is
// part of the FP8 code.
__device__ __forceinline__ float qdiv_fast(float x, float s, float inv)
{
    float q0 = x * inv;
    float r = __builtin_fmaf(-q0, s, x);
    float q = __builtin_fmaf(r, inv, q0);
    float a = __builtin_fabsf(q0);
    return (a < 0x1p120f && a != 0.0f) ? q : q0;
}

struct Divider {
    float s, inv;
    bool fast;
    __device__ __forceinline__ explicit Divider(float step)
    {
        s = step;
        inv = 1.0f / step;                    // IEEE division (correctly rounded)
        fast = step >= 0x1p-64f && step <= 0x1p64f;
    }
    __device__ __forceinline__ float operator()(float x) const
    {
        return fast ? qdiv_fast(x, s, inv) : x / s;
    }
    // The same with the path chosen at compile time (the caller tests
    // `fast` once for a whole loop).
    template <bool FAST> __device__ __forceinline__ float q(float x) const
    {
        return FAST ? qdiv_fast(x, s, inv) : x / s;
    }
};

// ---------------------------------------------------------------------------
// Saturating round-to-nearest-even encoders.  Each packs four quotients into
// one 32-bit word, code of element 0 in the low byte.
//
// FP8 uses the gfx950 converts (v_cvt_pk_fp8_f32 / v_cvt_pk_bf8_f32: OCP
// formats, round to nearest even, subnormals kept, sign of zero kept) after
// clamping to the largest finite value, so out-of-range values saturate
// instead of becoming NaN / inf.
template <int FMT>
__device__ __forceinline__ uint32_t encode4(float a, float b, float c, float d);

template <>
__device__ __forceinline__ uint32_t encode4<FMT_E4M3>(float a, float b, float c, float d)
{
    const float m = Fmt<FMT_E4M3>::qmax;
    a = __builtin_fminf(__builtin_fmaxf(a, -m), m);
    b = __builtin_fminf(__builtin_fmaxf(b, -m), m);
    c = __builtin_fminf(__builtin_fmaxf(c, -m), m);
    d = __builtin_fminf(__builtin_fmaxf(d, -m), m);
    // The first convert writes the low half of a register whose high half
    // the second one overwrites: start from a's bits, not a zeroed register.
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __builtin_bit_cast(int, a), false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

template <>
__device__ __forceinline__ uint32_t encode4<FMT_E5M2>(float a, float b, float c, float d)
{
    const float m = Fmt<FMT_E5M2>::qmax;
    a = __builtin_fminf(__builtin_fmaxf(a, -m), m);
    b = __builtin_fminf(__builtin_fmaxf(b, -m), m);
    c = __builtin_fminf(__builtin_fmaxf(c, -m), m);
    d = __builtin_fminf(__builtin_fmaxf(d, -m), m);
    // The first convert writes the low half of a register whose high half
    // the second one overwrites: start from a's bits, not a zeroed register.
    int w = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, __builtin_bit_cast(int, a), false);
    w = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, w, true);
    return (uint32_t)w;
}

// INT8: round half to even (v_rndne_f32), clamp to +-127, two's complement.
__device__ __forceinline__ uint32_t int8_byte(float v)
{
    v = __builtin_fminf(__builtin_fmaxf(__builtin_rintf(v), -127.0f), 127.0f);
    return (uint32_t)(int32_t)v & 0xFFu;
}

template <>
__device__ __forceinline__ uint32_t encode4<FMT_INT8>(float a, float b, float c, float d)
{
    return int8_byte(a) | (int8_byte(b) << 8) | (int8_byte(c) << 16) | (int8_byte(d) << 24);
}

template <int FMT>
__device__ __forceinline__ uint8_t encode1(float a)
{
    return (uint8_t)(encode4<FMT>(a, 0.0f, 0.0f, 0.0f) & 0xFFu);
}

// ---------------------------------------------------------------------------
// Exact FP8 decode by bit assembly (finite codes; NaN and inf codes are out
// of contract).  E4M3: exponent field 0 is m * 2^-9, else (1 + m/8) *
// 2^(e-7); E5M2: exponent field 0 is m * 2^-16, else (1 + m/4) * 2^(e-15).
template <int FMT> __device__ __forceinline__ float fp8_decode(uint32_t code);
template <> __device__ __forceinline__ float fp8_decode<FMT_E4M3>(uint32_t code)
{
    const uint32_t s = (code & 0x80u) << 24, e = (code >> 3) & 0xFu, m = code & 7u;
    const float mag = e == 0 ? (float)m * 0x1p-9f : __uint_as_float(((e + 120u) << 23) | (m << 20));
    return __uint_as_float(__float_as_uint(mag) | s);
}
template <> __device__ __forceinline__ float fp8_decode<FMT_E5M2>(uint32_t code)
{
    const uint32_t s = (code & 0x80u) << 24, e = (code >> 2) & 0x1Fu, m = code & 3u;
    const float mag = e == 0 ? (float)m * 0x1p-16f : __uint_as_float(((e + 112u) << 23) | (m << 21));
    return __uint_as_float(__float_as_uint(mag) | s);
}

// ---------------------------------------------------------------------------
// Wave64 / workgroup reductions of unsigned maxima.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        uint32_t o = (uint32_t)__shfl_xor((int)v, off, 64);
        v = o > v ? o : v;
    }
    return v;
}

// Block-wide maximum; every thread receives the result.  `red` must hold
// one word per wave of the block.
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t *red)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nwaves = (blockDim.x + 63) >> 6;
    v = wave_max_u32(v);
    if (lane == 0) red[wave] = v;
    __syncthreads();
    uint32_t r = 0;
    for (int i = 0; i < nwaves; ++i) r = red[i] > r ? red[i] : r;
    __syncthreads();
    return r;
}

// ---------------------------------------------------------------------------
// Last-workgroup election over a 2-word workspace slot {amax bits, counter}.
//
// Every workgroup folds its maximum into slot[0] with a device-scope atomic
// max and, once that has returned, increments slot[1]; the workgroup that
// sees the count reach `count` - 1 is the last one and reads the maximum
// back with one more read-modify-write issued after its increment returned.
// Device-scope read-modify-writes are performed at the memory side, one
// order per address for every XCD, and each one here is issued only after
// the previous one of the same workgroup has completed, so the last read
// comes after every workgroup's max.  All of them are relaxed: no
// workgroup's other stores are ordered by the election, only the maximum
// that travels through the atomics is, and no L2 is written back or
// invalidated (an acquire-release increment would do both, which costs
// the streaming kernels a write-back of their dirty output per workgroup).
// The last workgroup leaves the slot zeroed for the next call (the kernel's
// end makes those stores visible to later launches), so no clearing launch
// is ever needed.  Only thread 0 of each workgroup calls this; it returns
// true (and *result) in the last.
//
// Cost: read-modify-writes on one address are serialized by the memory
// system (about 10 ns each on MI355X), so the grids that elect stay at a
// few hundred workgroups finishing together.  `count` is the number of
// workgroups that take part (a grid row, when the rows of a grid are
// independent elections).
__device__ __forceinline__ uint32_t opaque_u32(uint32_t v)
{
    asm volatile("v_mov_b32 %0, %1" : "=v"(v) : "v"(v));    // hides the value from the compiler
    return v;
}

__device__ __forceinline__ bool elect_last_max_n(uint32_t *slot, uint32_t block_max, uint32_t *result,
                                                 uint32_t count)
{
    const uint32_t before = __hip_atomic_fetch_max(&slot[0], block_max, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("" : : "v"(before) : "memory");               // the max has returned
    const uint32_t prev = __hip_atomic_fetch_add(&slot[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("" : : "v"(prev) : "memory");                 // the increment has returned
    if (prev != count - 1) return false;
    // max with an opaque zero: a read-modify-write the compiler cannot turn into a load
    const uint32_t m = __hip_atomic_fetch_max(&slot[0], opaque_u32(0u), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("" : : "v"(m) : "memory");
    *result = m;
    __hip_atomic_store(&slot[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&slot[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
}

// The election over the whole grid.
__device__ __forceinline__ bool elect_last_max(uint32_t *slot, uint32_t block_max, uint32_t *result)
{
    return elect_last_max_n(slot, block_max, result, gridDim.x * gridDim.y);
}

}  // namespace ql
