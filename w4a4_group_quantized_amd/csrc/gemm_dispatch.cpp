// Kernel choice for apex4_gemm_w4a4.  Few rows: the call is bound by reading
// the packed weights once; up to 2 rows the dot8 kernel streams whole weight
// rows per wave, up to 16 the LDS-streaming MFMA kernel, up to 64 its variant
// with K outside the column blocks (the skinny kernel, feeding the matrix
// units from global memory, covers the group modes those lack).  Otherwise the call is
// compute-bound and one of the tiled kernels runs (the ping-pong one for
// groups of 64, 128, 256 or one group over K, the step-major one for groups
// of 32 and for mixed mode with activation groups of 32 or 64).
#include "internal.h"

namespace apex4 {

GemmKernel gemm_kernel(const GemmProblem& p)
{
    if (p.M <= 2 && gemv_supports(p)) return GemmKernel::Gemv;
#ifndef APEX4_NO_STREAM
    if (stream_supports(p)) return GemmKernel::Stream;
#endif
    if (gemv_supports(p)) return GemmKernel::Gemv;
#ifndef APEX4_NO_KOUTER
    if (kouter_supports(p)) return GemmKernel::Kouter;
#endif
    if (skinny_supports(p)) return GemmKernel::Skinny;
#ifndef APEX4_NO_PINGPONG
    if (pingpong_supports(p)) return GemmKernel::Pingpong;
#endif
    return GemmKernel::Tiled;
}

size_t gemm_workspace_bytes(const GemmProblem& p)
{
    // the K-outer and ping-pong kernels' K splits
    switch (gemm_kernel(p)) {
    case GemmKernel::Kouter: return kouter_workspace_bytes(p);
    case GemmKernel::Pingpong: return pingpong_split(p).bytes;
    default: return 0;
    }
}

hipError_t launch_gemm(const GemmProblem& p, hipStream_t stream)
{
    switch (gemm_kernel(p)) {
    case GemmKernel::Gemv: return launch_gemm_gemv(p, stream);
    case GemmKernel::Stream: return launch_gemm_stream(p, stream);
    case GemmKernel::Kouter: return launch_gemm_kouter(p, stream);
    case GemmKernel::Skinny: return launch_gemm_skinny(p, stream);
    case GemmKernel::Pingpong: return launch_gemm_pingpong(p, stream);
    default: return launch_gemm_tiled(p, stream);
    }
}

}  // namespace apex4
