// noalloc.hip -- ql_linear_forward_noalloc: ql_linear_forward with its
// workspace in a file-scope device array instead of caller memory, for
// callers that cannot allocate device memory (code under HIP graph
// capture, serving loops, harnesses that forbid hipMalloc).
//
// The array is the same workspace layout ql_linear_forward uses
// (internal.hpp): the counter slots of the three last-workgroup elections
// (quantize of x, of w, the GEMM's out_amax), then the per-workgroup
// maxima.  Its size does not depend on the problem size: the whole-tensor
// quantize grid is capped at 256 workgroups, and a GEMM grid with more
// workgroups than the maxima area holds falls back to the election.  Each
// GPU holds one copy, at its own address, until the process ends.
#include <mutex>

#include "internal.hpp"
#include "qlinear.h"

namespace {

constexpr int64_t SCRATCH_BYTES = ql::WS_BYTES;
static_assert(SCRATCH_BYTES % 256 == 0, "the scratch array is a whole number of 256-byte slots");

// Device memory of the allocation-free entry point.  Host code never
// passes this name to a kernel or a copy: on the host it is only a handle,
// whose device address hipGetSymbolAddress gives per device.
static __device__ __align__(256) uint8_t scratch[SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void *g_scratch[MAX_DEVICES];   // scratch's address on each device, once looked up

// The address of scratch on the current device, looked up (with that
// device current) on the first call for the device.
hipError_t scratch_on_current_device(void **out, int *dev_out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    *dev_out = dev;
    return hipSuccess;
}

}  // namespace

extern "C" ql_status ql_linear_forward_noalloc(const void *x, ql_dtype x_dt, int64_t M, int64_t K,
                                               const void *w, int64_t N,
                                               const void *bias, ql_dtype bias_dt, ql_qfmt fmt,
                                               const float *sx_in, const float *sw_in,
                                               void *out, ql_dtype out_dt, const float *out_scale, float *out_amax,
                                               void *x_q, float *sx, float *amax_x,
                                               void *w_q, float *sw, float *amax_w, void *stream)
{
    static const char *what = "linear_forward_noalloc";
    void *ws = nullptr;
    int dev = -1;
    hipError_t e = scratch_on_current_device(&ws, &dev);
    if (e != hipSuccess) return (ql_status)ql::report_error(QL_ERR_HIP, what, hipGetErrorString(e));
    if (stream) {
        // The scratch address is the current device's: the stream must run
        // there too.
        int sdev = -1;
        e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev);
        if (e != hipSuccess) return (ql_status)ql::report_error(QL_ERR_HIP, what, hipGetErrorString(e));
        if (sdev != dev)
            return (ql_status)ql::report_error(QL_ERR_VALUE, what, "the stream belongs to another device than the "
                                                                   "current one");
    }
    // Validation first; then the counter slots are cleared (a fill kernel
    // on the caller's stream) and the work enqueued after it.
    return (ql_status)ql::linear_forward_ws(x, x_dt, M, K, w, N, bias, bias_dt, fmt, sx_in, sw_in, out, out_dt,
                                            out_scale, out_amax, x_q, sx, amax_x, w_q, sw, amax_w, ws, true, stream);
}
