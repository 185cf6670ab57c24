// Kernel choice for apex4_gemm_w4a4.  Few rows: the call is bound by reading
// the packed weights once, and the skinny kernel spreads that stream over all
// CUs; otherwise the call is compute-bound and one of the tiled kernels runs
// (the ping-pong one for groups of 128 or more, the step-major one for 32
// and 64).
#include "internal.h"

namespace apex4 {

hipError_t launch_gemm(const GemmProblem& p, hipStream_t stream)
{
    if (skinny_supports(p)) return launch_gemm_skinny(p, stream);
#ifndef APEX4_NO_PINGPONG
    if (pingpong_supports(p)) return launch_gemm_pingpong(p, stream);
#endif
    return launch_gemm_tiled(p, stream);
}

}  // namespace apex4
