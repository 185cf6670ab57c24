// apex4_gemm_w4a4_noalloc (include/apex4.h): the GEMM for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  The only scratch memory the GEMM kernels
// use is the fp32 partial results of their K splits (the ping-pong kernel's
// partial last round of tiles, the K-outer kernel's two halves); here it is
// the library's own fixed array instead of a caller workspace.
//
// The array lives in device memory of every GPU the library runs on, from
// module load to process end.  Host code never passes the array's name to a
// kernel (on the host that name is only a stand-in): once per device, with the
// device current, hipGetSymbolAddress gives the device address, which is kept
// per device and passed as the workspace.  The splits overwrite every partial
// value they later read, so nothing needs clearing between calls; calls that
// overlap on one GPU share the array and race.
#include <mutex>

#include "apex4.h"
#include "internal.h"

namespace apex4 {
namespace {

// Largest partial-result set: the ping-pong split writes at most one 256x128
// fp32 tile per compute unit (32 MiB on 256 compute units); the K-outer split
// 2 x M x N fp32 values (M <= 64, N <= 8192: at most 4 MiB).
constexpr size_t kScratchBytes = APEX4_NOALLOC_MAX_WORKSPACE;

__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;

struct ScratchTable {
    std::mutex mu;
    void* ptr[kMaxDevices] = {};
};

ScratchTable& table()
{
    static ScratchTable t;
    return t;
}

// The device address of this device's scratch array (looked up once per
// device, with that device current), or null with the HIP error in *err.
void* scratch_of_current_device(hipError_t* err)
{
    *err = hipSuccess;
    int dev = -1;
    if ((*err = hipGetDevice(&dev)) != hipSuccess) return nullptr;
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    ScratchTable& t = table();
    std::lock_guard<std::mutex> lock(t.mu);
    if (t.ptr[dev] == nullptr) {
        void* p = nullptr;
        if ((*err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return nullptr;
        t.ptr[dev] = p;
    }
    return t.ptr[dev];
}

}  // namespace
}  // namespace apex4

extern "C" {

apex4_status apex4_gemm_w4a4_noalloc(const void* qa_u8, const float* s_a, int32_t group_a, const void* qw_u8,
                                     const float* s_w, int32_t group_w, int64_t M, int64_t N, int64_t K,
                                     void* y_f16, float* y_f32, void* stream)
{
    // the shape's workspace must fit the array; the size query itself checks
    // nothing else, the call below does every check of apex4_gemm_w4a4
    const size_t need = apex4_gemm_workspace_size(M, N, K, group_a, group_w);
    if (need > apex4::kScratchBytes) return APEX4_ERR_WORKSPACE;
    void* ws = nullptr;
    if (need > 0) {
        hipError_t err;
        ws = apex4::scratch_of_current_device(&err);
        if (ws == nullptr) return APEX4_ERR_HIP;
    }
    return apex4::gemm_checked(qa_u8, s_a, group_a, qw_u8, s_w, group_w, M, N, K, y_f16, y_f32, 0, 1, M, nullptr,
                               ws, need > 0 ? apex4::kScratchBytes : 0, stream);
}

}  // extern "C"
