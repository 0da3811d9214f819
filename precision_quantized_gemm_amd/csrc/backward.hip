// backward.hip -- grad_bias of the quantized linear layer's backward: the
// column sums of the BF16 output gradient g [M, N] (AstrAI ops/fp8.py
// linear_backward_fp8 returns grad_bias beside dX and dW).
//
// One workgroup owns 64 columns; its 16 waves each sum every 16th row of
// those columns (a wave reads 128 contiguous bytes per row), and the 16
// partial sums of a column are added in a fixed order, so the result does
// not depend on scheduling.  FP32 accumulation: M/16 + 16 additions per
// column.
#include "qdev.hpp"
#include "internal.hpp"

namespace ql {

constexpr int CS_COLS = 64, CS_GROUPS = 16;

__global__ __launch_bounds__(CS_COLS * CS_GROUPS) void col_sum_bf16(const uint16_t *g, int64_t M, int64_t N,
                                                                   int64_t ldg, float *out)
{
    const int cx = threadIdx.x % CS_COLS, ry = threadIdx.x / CS_COLS;
    const int64_t col = (int64_t)blockIdx.x * CS_COLS + cx;
    float s = 0.0f;
    if (col < N)
        for (int64_t r = ry; r < M; r += CS_GROUPS) s += __uint_as_float((uint32_t)g[r * ldg + col] << 16);
    __shared__ float part[CS_GROUPS][CS_COLS + 1];
    part[ry][cx] = s;
    __syncthreads();
    if (ry == 0 && col < N) {
        float t = 0.0f;
#pragma unroll
        for (int i = 0; i < CS_GROUPS; ++i) t += part[i][cx];
        out[col] = t;
    }
}

hipError_t launch_col_sum_bf16(const void *g, int64_t M, int64_t N, int64_t ldg, float *out, hipStream_t s)
{
    if (N == 0) return hipSuccess;
    const int64_t blocks = (N + CS_COLS - 1) / CS_COLS;
    hipLaunchKernelGGL(col_sum_bf16, dim3((unsigned)blocks), dim3(CS_COLS * CS_GROUPS), 0, s,
                       static_cast<const uint16_t *>(g), M, N, ldg, out);
    return hipGetLastError();
}

}  // namespace ql
