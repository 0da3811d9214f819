// backward.hip -- grad_bias of the quantized linear layer's backward: the
// column sums of the BF16 output gradient g [M, N] (AstrAI ops/fp8.py
// linear_backward_fp8 returns grad_bias beside dX and dW).
//
// Two deterministic stages, with a summation order fixed by (M, N) alone:
//   col_sum_part  grid (column blocks of 512, S row splits).  Each lane owns
//                 8 consecutive columns (one 16-byte load of a row); the 4
//                 waves of a workgroup take every 4th row of the split, and
//                 their sums are added in wave order.  With S = 1 the result
//                 goes straight to grad_bias; else to partial row s.
//   col_sum_final adds the S partial rows of each column in split order.
// FP32 accumulation; a column's sum passes through at most
// ceil(ceil(M/S)/4) + 3 + S additions.
#include "qdev.hpp"
#include "internal.hpp"

namespace ql {

constexpr int CS_THREADS = 256;                 // 4 waves
constexpr int CS_VEC = 8;                       // columns per lane
constexpr int CS_COLS = 64 * CS_VEC;            // columns per workgroup
constexpr int CS_UNROLL = 4;                    // rows in flight per lane
constexpr int CS_MAX_SPLITS = 32;

template <bool VEC>
__global__ __launch_bounds__(CS_THREADS) void col_sum_part(const uint16_t *g, int64_t M, int64_t N, int64_t ldg,
                                                           int64_t rows_per_split, float *dst)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t col0 = (int64_t)blockIdx.x * CS_COLS + lane * CS_VEC;
    const int64_t r_begin = (int64_t)blockIdx.y * rows_per_split;
    const int64_t r_end = r_begin + rows_per_split < M ? r_begin + rows_per_split : M;
    float acc[CS_VEC];
#pragma unroll
    for (int e = 0; e < CS_VEC; ++e) acc[e] = 0.0f;

    auto load_row = [&](int64_t r, uint32_t (&w)[4]) {
        const uint16_t *src = g + r * ldg + col0;
        if (VEC) {
            if (col0 < N) {
                const uint4 v = *reinterpret_cast<const uint4 *>(src);
                w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
            } else {
                w[0] = w[1] = w[2] = w[3] = 0u;
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t lo = col0 + 2 * e < N ? src[2 * e] : 0u;
                const uint32_t hi = col0 + 2 * e + 1 < N ? src[2 * e + 1] : 0u;
                w[e] = lo | (hi << 16);
            }
        }
    };
    auto add_row = [&](const uint32_t (&w)[4]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[2 * e] += bf16_lo(w[e]);
            acc[2 * e + 1] += bf16_hi(w[e]);
        }
    };

    // Rows r_begin + wave + 4i, four loads in flight, added in row order.
    int64_t r = r_begin + wave;
    for (; r + 4 * (CS_UNROLL - 1) < r_end; r += 4 * CS_UNROLL) {
        uint32_t w[CS_UNROLL][4];
#pragma unroll
        for (int u = 0; u < CS_UNROLL; ++u) load_row(r + 4 * u, w[u]);
#pragma unroll
        for (int u = 0; u < CS_UNROLL; ++u) add_row(w[u]);
    }
    for (; r < r_end; r += 4) {
        uint32_t w[4];
        load_row(r, w);
        add_row(w);
    }

    __shared__ float part[4][CS_VEC][64 + 1];
#pragma unroll
    for (int e = 0; e < CS_VEC; ++e) part[wave][e][lane] = acc[e];
    __syncthreads();
    if (wave == 0) {
        float* out = dst + (int64_t)blockIdx.y * N;
#pragma unroll
        for (int e = 0; e < CS_VEC; ++e) {
            const float t = ((part[0][e][lane] + part[1][e][lane]) + part[2][e][lane]) + part[3][e][lane];
            if (col0 + e < N) out[col0 + e] = t;
        }
    }
}

__global__ __launch_bounds__(256) void col_sum_final(const float *part, int64_t N, int splits, float *out)
{
    const int64_t col = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (col >= N) return;
    float v[CS_MAX_SPLITS];                        // every load in flight, then added in split order
#pragma unroll
    for (int s = 0; s < CS_MAX_SPLITS; ++s) v[s] = s < splits ? part[(int64_t)s * N + col] : 0.0f;
    float t = v[0];
#pragma unroll
    for (int s = 1; s < CS_MAX_SPLITS; ++s)
        if (s < splits) t += v[s];
    out[col] = t;
}

int col_sum_splits(int64_t M, int64_t N)
{
    const int64_t blocks = (N + CS_COLS - 1) / CS_COLS;
    int64_t s = (512 + blocks - 1) / blocks;                  // about 512 workgroups
    const int64_t by_rows = (M + 4 * CS_UNROLL - 1) / (4 * CS_UNROLL);
    const int64_t by_ws = WS_PART_BYTES / (4 * (N > 0 ? N : 1));
    if (s > CS_MAX_SPLITS) s = CS_MAX_SPLITS;
    if (s > by_rows) s = by_rows;
    if (s > by_ws) s = by_ws;
    return s < 1 ? 1 : (int)s;
}

hipError_t launch_col_sum_bf16(const void *g, int64_t M, int64_t N, int64_t ldg, float *out, float *partials,
                               hipStream_t s)
{
    if (N == 0) return hipSuccess;
    const int splits = col_sum_splits(M, N);
    const int64_t rows_per_split = splits > 1 ? (M + splits - 1) / splits : (M > 0 ? M : 1);
    const dim3 grid((unsigned)((N + CS_COLS - 1) / CS_COLS), (unsigned)splits);
    float *dst = splits > 1 ? partials : out;
    const uint16_t *gp = static_cast<const uint16_t *>(g);
    const bool vec = (reinterpret_cast<uintptr_t>(g) & 15u) == 0 && N % CS_VEC == 0 && ldg % CS_VEC == 0;
    if (vec) hipLaunchKernelGGL(col_sum_part<true>, grid, dim3(CS_THREADS), 0, s, gp, M, N, ldg, rows_per_split, dst);
    else hipLaunchKernelGGL(col_sum_part<false>, grid, dim3(CS_THREADS), 0, s, gp, M, N, ldg, rows_per_split, dst);
    if (splits > 1)
        hipLaunchKernelGGL(col_sum_final, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, s, partials, N, splits,
                           out);
    return hipGetLastError();
}

}  // namespace ql
