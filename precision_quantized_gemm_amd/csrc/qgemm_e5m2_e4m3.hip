// qgemm_e5m2_e4m3.hip -- instantiations of the scaled GEMM for A in FMT_E5M2 and B in
// FMT_E4M3 (one file per format pair so the build compiles them in parallel).
#include "qgemm_impl.hpp"
#include "qgemm_nt.hpp"
#include "qgemm_dl.hpp"
#include "qgemm_pipe.hpp"

namespace ql {

hipError_t launch_qgemm_e5m2_e4m3(const GemmParams &p, int a_mn, int b_mn, hipStream_t s)
{
    return launch_formats<FMT_E5M2, FMT_E4M3>(p, a_mn, b_mn, s);
}

}  // namespace ql
