// Kernel choice for apex4_gemm_w4a4.  Few rows: the call is bound by reading
// the packed weights once, and the skinny kernel spreads that stream over all
// CUs; otherwise the call is compute-bound and the tiled kernel runs.
#include "internal.h"

namespace apex4 {

hipError_t launch_gemm(const GemmProblem& p, hipStream_t stream)
{
    if (skinny_supports(p)) return launch_gemm_skinny(p, stream);
    return launch_gemm_tiled(p, stream);
}

}  // namespace apex4
