// measure.hip -- ql_stream_probe (include/qlinear_measure.h): the quantize
// cast's memory traffic without its arithmetic, for the memory system's
// ceiling on that access pattern.  Same grid shape as the whole-tensor
// quantize kernels (at most 256 workgroups of 1024 threads, four units in
// flight per lane, units strided by the grid), 16-byte non-temporal loads
// and plain stores.
#include "internal.hpp"
#include "qlinear_measure.h"

namespace {

constexpr int PROBE_THREADS = 1024;
constexpr int PROBE_MAX_BLOCKS = 256;
constexpr int PROBE_UNROLL = 4;

__device__ __forceinline__ uint4 xor4(uint4 a, uint4 b) { return make_uint4(a.x ^ b.x, a.y ^ b.y, a.z ^ b.z, a.w ^ b.w); }

// Non-temporal 16-byte loads, plain stores: the fastest of the four
// combinations for the 2:1 mix (71.0 us for 256 MiB read + 128 MiB written,
// against 77.2 us with plain loads), as in the single-pass delayed cast;
// read-only runs the same with either load.
typedef unsigned int u32v4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const uint4 *p)
{
    const u32v4 x = __builtin_nontemporal_load(reinterpret_cast<const u32v4 *>(p));
    return make_uint4(x.x, x.y, x.z, x.w);
}

// Unit u: 32 bytes at src[2u], src[2u+1] (16-byte words); WRITE stores
// their XOR at dst[u], otherwise the thread folds it into one word.
template <bool WRITE>
__global__ __launch_bounds__(PROBE_THREADS) void stream_probe_kernel(const uint4 *src, int64_t n_units, uint4 *dst,
                                                                     uint32_t *sink)
{
    const int64_t gtid = (int64_t)blockIdx.x * PROBE_THREADS + threadIdx.x;
    const int64_t gstride = (int64_t)gridDim.x * PROBE_THREADS;
    uint32_t fold = 0;
    int64_t u = gtid;
    for (; u + (PROBE_UNROLL - 1) * gstride < n_units; u += PROBE_UNROLL * gstride) {
        uint4 a[PROBE_UNROLL], b[PROBE_UNROLL];
#pragma unroll
        for (int j = 0; j < PROBE_UNROLL; ++j) {
            a[j] = load_stream(src + 2 * (u + j * gstride));
            b[j] = load_stream(src + 2 * (u + j * gstride) + 1);
        }
#pragma unroll
        for (int j = 0; j < PROBE_UNROLL; ++j) {
            const uint4 x = xor4(a[j], b[j]);
            if (WRITE) dst[u + j * gstride] = x;
            else fold ^= x.x ^ x.y ^ x.z ^ x.w;
        }
    }
    for (; u < n_units; u += gstride) {
        const uint4 x = xor4(load_stream(src + 2 * u), load_stream(src + 2 * u + 1));
        if (WRITE) dst[u] = x;
        else fold ^= x.x ^ x.y ^ x.z ^ x.w;
    }
    if (!WRITE) sink[gtid] = fold;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" ql_status ql_stream_probe(const void *src, int64_t n_units, void *dst, void *sink, void *stream)
{
    static const char *what = "stream_probe";
    if (n_units < 0) return (ql_status)ql::report_error(QL_ERR_VALUE, what, "negative n_units");
    if (n_units == 0) return QL_OK;
    if (!src) return (ql_status)ql::report_error(QL_ERR_NULL, what, "src is required");
    if ((dst == nullptr) == (sink == nullptr))
        return (ql_status)ql::report_error(QL_ERR_VALUE, what, "exactly one of dst and sink must be given");
    if (!aligned16(src) || !aligned16(dst) || !aligned16(sink))
        return (ql_status)ql::report_error(QL_ERR_VALUE, what, "buffers must be 16-byte aligned");
    int64_t blocks = (n_units + PROBE_THREADS - 1) / PROBE_THREADS;
    if (blocks > PROBE_MAX_BLOCKS) blocks = PROBE_MAX_BLOCKS;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const uint4 *in = static_cast<const uint4 *>(src);
    if (dst)
        hipLaunchKernelGGL(stream_probe_kernel<true>, dim3((unsigned)blocks), dim3(PROBE_THREADS), 0, s, in, n_units,
                           static_cast<uint4 *>(dst), nullptr);
    else
        hipLaunchKernelGGL(stream_probe_kernel<false>, dim3((unsigned)blocks), dim3(PROBE_THREADS), 0, s, in,
                           n_units, nullptr, static_cast<uint32_t *>(sink));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (ql_status)ql::report_error(QL_ERR_HIP, what, hipGetErrorString(e));
    return QL_OK;
}
