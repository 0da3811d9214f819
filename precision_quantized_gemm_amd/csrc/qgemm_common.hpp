// qgemm_common.hpp -- what the general GEMM kernel and the pipelined FP8
// kernel share: operand vector types, the workgroup size, buffer-load
// constants, the fused epilogue and the XCD-aware tile order.
//
//   out[m, n] = (sum_k A[m, k] * B[n, k]) * sa[m|0] * sb[n|0] (+ bias[n])
//
// AstrAI ops/fp8.py @5e76fbd: fp8_gemm / mm_fp8 (a @ b * (sa*sb), FP32
// accumulation, BF16 or E4M3 output where E4M3 divides by out_scale) and
// linear_forward_fp8 (bias fused into the GEMM epilogue); scmp_kernels
// README "API" (a @ b.T, per-row scales).
#pragma once

#include "qdev.hpp"
#include "internal.hpp"

namespace ql {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int GEMM_THREADS = 256;
constexpr int GEMM_GM = 8;   // tile-rows per group in the tile order

constexpr uint32_t BUF_OOB = 0x80000000u;
constexpr int BUF_WORD3 = 0x00020000;   // gfx9 raw-buffer descriptor word 3

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Fused epilogue for 4 consecutive outputs of one row:
//   v = acc * sa[row|0] * sb[col|0] (+ bias[col]), then the output cast.
// Per-tensor scales fold into one FP32 product sa*sb (either order of the
// two multiplies is within the float acceptance bound).  E4M3 output
// multiplies by RN(1/out_scale): its result differs from the correctly
// rounded quotient by at most one FP32 rounding, which the FP8 acceptance
// set allows for; with per-tensor scales and no bias the accumulator is
// multiplied once by RN(sa*sb * RN(1/out_scale)) instead (the same number
// of roundings).
struct Epilogue {
    const GemmParams &p;
    float inv_os;       // RN(1 / out_scale) for E4M3 output
    float s_ab;         // sa[0] * sb[0] when both are per tensor
    float s_out;        // RN(s_ab * inv_os): E4M3 output, per-tensor scales, no bias
    bool per_tensor;
    __device__ __forceinline__ explicit Epilogue(const GemmParams &pp) : p(pp)
    {
        inv_os = pp.out_dt == DT_E4M3 ? 1.0f / pp.out_scale[0] : 1.0f;
        per_tensor = pp.sa_group == 0 && pp.sb_group == 0;
        s_ab = (per_tensor && pp.out_dt != DT_INT32) ? pp.sa[0] * pp.sb[0] : 1.0f;
        s_out = s_ab * inv_os;
    }

    __device__ __forceinline__ float bias_at(int64_t col) const
    {
        if (p.bias_dt == DT_FP32) return static_cast<const float *>(p.bias)[col];
        if (p.bias_dt == DT_BF16) return __uint_as_float((uint32_t)static_cast<const uint16_t *>(p.bias)[col] << 16);
        if (p.bias_dt == BIAS_Q_E4M3)
            return fp8_decode<FMT_E4M3>(static_cast<const uint8_t *>(p.bias)[col]) * p.bias_scale[0];
        if (p.bias_dt == BIAS_Q_E5M2)
            return fp8_decode<FMT_E5M2>(static_cast<const uint8_t *>(p.bias)[col]) * p.bias_scale[0];
        return 0.0f;
    }

    template <bool INT_ACC>
    __device__ __forceinline__ uint32_t store4(uint4 w, int64_t row, int64_t col, uint32_t vmax) const
    {
        const uint32_t raw[4] = {w.x, w.y, w.z, w.w};
        const int n = p.N - col < 4 ? (int)(p.N - col) : 4;
        const int64_t o = row * p.ldo + col;
        if (p.out_dt == DT_INT32) {
            int32_t *out = static_cast<int32_t *>(p.out) + o;
            if (n == 4 && p.out_vec4) *reinterpret_cast<uint4 *>(out) = w;
            else for (int e = 0; e < n; ++e) out[e] = (int32_t)raw[e];
            return vmax;
        }
        float v[4];
        if (per_tensor) {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = (INT_ACC ? (float)(int32_t)raw[e] : __uint_as_float(raw[e])) * s_ab;
        } else {
            const float s_row = p.sa[p.sa_div((uint32_t)(p.row_base + row))];
            const uint32_t c0 = (uint32_t)(p.col_base + col);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float a = INT_ACC ? (float)(int32_t)raw[e] : __uint_as_float(raw[e]);
                v[e] = a * s_row * p.sb[p.sb_div(c0 + (uint32_t)(e < n ? e : 0))];
            }
        }
        if (p.bias_dt >= 0) {
            if (n == 4 && p.bias_dt == DT_FP32 && (col & 3) == 0 && p.out_vec4) {
                const float4 b = *reinterpret_cast<const float4 *>(static_cast<const float *>(p.bias) + col);
                v[0] += b.x; v[1] += b.y; v[2] += b.z; v[3] += b.w;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] += bias_at(col + (e < n ? e : 0));
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (e < n) { const uint32_t b = absbits_f32(v[e]); vmax = b > vmax ? b : vmax; }
        if (p.out_dt == DT_BF16) {
            uint16_t h[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) h[e] = __builtin_bit_cast(uint16_t, (__bf16)v[e]);
            uint16_t *out = static_cast<uint16_t *>(p.out) + o;
            if (n == 4 && p.out_vec4)
                *reinterpret_cast<uint2 *>(out) = make_uint2(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16));
            else for (int e = 0; e < n; ++e) out[e] = h[e];
        } else if (p.out_dt == DT_FP32) {
            float *out = static_cast<float *>(p.out) + o;
            if (n == 4 && p.out_vec4) *reinterpret_cast<float4 *>(out) = make_float4(v[0], v[1], v[2], v[3]);
            else for (int e = 0; e < n; ++e) out[e] = v[e];
        } else {
            // Per-tensor scales and no bias: one multiply of the accumulator
            // by RN(sa*sb / out_scale); otherwise v times RN(1 / out_scale).
            float u[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                u[e] = (per_tensor && p.bias_dt < 0)
                           ? (INT_ACC ? (float)(int32_t)raw[e] : __uint_as_float(raw[e])) * s_out
                           : v[e] * inv_os;
            const uint32_t c = encode4<FMT_E4M3>(u[0], u[1], u[2], u[3]);
            uint8_t *out = static_cast<uint8_t *>(p.out) + o;
            if (n == 4 && p.out_vec4) *reinterpret_cast<uint32_t *>(out) = c;
            else for (int e = 0; e < n; ++e) out[e] = (uint8_t)(c >> (8 * e));
        }
        return vmax;
    }
};

// End of a GEMM workgroup's out_amax: the workgroup maximum goes to its
// own slot of p.amax_part (reduced by a small kernel after the GEMM), or,
// without that array, into the last-workgroup election (grids of one wave:
// no launch after the GEMM).
__device__ __forceinline__ void gemm_publish_amax(const GemmParams &p, uint32_t vmax, uint32_t *red)
{
    vmax = block_max_u32(vmax, red);
    if (threadIdx.x == 0) {
        if (p.amax_part) {
            p.amax_part[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] = vmax;
        } else {
            uint32_t bits;
            if (elect_last_max(p.ws, vmax, &bits)) p.out_amax[0] = __uint_as_float(bits);
        }
    }
}

// Linear tile id -> (tile_m, tile_n): XCD-contiguous, then grouped.  Ids
// that are equal mod 8 run on one XCD when the launch hands consecutive
// workgroups to consecutive XCDs (a persistent grid must be a multiple of 8
// for its ids id, id + grid, ... to keep that property).
__device__ __forceinline__ void tile_coords_of(int id, int tiles_m, int tiles_n, int &tm, int &tn)
{
    const int total = tiles_m * tiles_n;
    int t = id;
    if ((total & 7) == 0) t = (t & 7) * (total >> 3) + (t >> 3);
    const int per_group = GEMM_GM * tiles_n;
    const int first_m = (t / per_group) * GEMM_GM;
    const int gsize = tiles_m - first_m < GEMM_GM ? tiles_m - first_m : GEMM_GM;
    const int in_group = t - (t / per_group) * per_group;
    tm = first_m + in_group % gsize;
    tn = in_group / gsize;
}

__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int &tm, int &tn)
{
    tile_coords_of((int)blockIdx.x, tiles_m, tiles_n, tm, tn);
}

}  // namespace ql
