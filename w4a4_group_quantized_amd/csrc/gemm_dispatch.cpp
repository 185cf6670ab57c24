// Kernel choice for apex4_gemm_w4a4.  Few rows: the call is bound by reading
// the packed weights once; up to 2 rows the dot8 kernel streams whole weight
// rows per wave, up to 16 the LDS-streaming MFMA kernel, up to 64 its variant
// with K outside the column blocks (the skinny kernel, feeding the matrix
// units from global memory, covers the group modes those lack).  Otherwise the call is
// compute-bound and one of the tiled kernels runs (the ping-pong one for
// groups of 128 or one group over K, the step-major one for the other group
// sizes).
#include "internal.h"

namespace apex4 {

size_t gemm_workspace_bytes(const GemmProblem& p)
{
    // mirrors the order of launch_gemm: the K-outer and ping-pong kernels' K splits
    if (p.M <= 2 && gemv_supports(p)) return 0;
#ifndef APEX4_NO_STREAM
    if (stream_supports(p)) return 0;
#endif
    if (gemv_supports(p)) return 0;
#ifndef APEX4_NO_KOUTER
    if (kouter_supports(p)) return kouter_workspace_bytes(p);
#endif
    if (skinny_supports(p)) return 0;
#ifndef APEX4_NO_PINGPONG
    if (pingpong_supports(p)) return pingpong_split(p).bytes;
#endif
    return 0;
}

hipError_t launch_gemm(const GemmProblem& p, hipStream_t stream)
{
    if (p.M <= 2 && gemv_supports(p)) return launch_gemm_gemv(p, stream);
#ifndef APEX4_NO_STREAM
    if (stream_supports(p)) return launch_gemm_stream(p, stream);
#endif
    if (gemv_supports(p)) return launch_gemm_gemv(p, stream);
#ifndef APEX4_NO_KOUTER
    if (kouter_supports(p)) return launch_gemm_kouter(p, stream);
#endif
    if (skinny_supports(p)) return launch_gemm_skinny(p, stream);
#ifndef APEX4_NO_PINGPONG
    if (pingpong_supports(p)) return launch_gemm_pingpong(p, stream);
#endif
    return launch_gemm_tiled(p, stream);
}

}  // namespace apex4
