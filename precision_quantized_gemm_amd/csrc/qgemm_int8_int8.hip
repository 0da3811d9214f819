// qgemm_int8_int8.hip -- instantiations of the scaled GEMM for A in FMT_INT8 and B in
// FMT_INT8 (one file per format pair so the build compiles them in parallel).
#include "qgemm_impl.hpp"
#include "qgemm_nt.hpp"
#include "qgemm_dl.hpp"
#include "qgemm_pipe.hpp"

namespace ql {

hipError_t launch_qgemm_int8_int8(const GemmParams &p, int a_mn, int b_mn, hipStream_t s)
{
    return launch_formats<FMT_INT8, FMT_INT8>(p, a_mn, b_mn, s);
}

}  // namespace ql
