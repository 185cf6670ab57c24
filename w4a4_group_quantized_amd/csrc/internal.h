// Internal launchers behind the C ABI in include/apex4.h.  Arguments are
// already validated by the caller (api.cpp); each returns hipGetLastError()
// after its launches.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace apex4 {

// Per-group symmetric INT4 quantization of fp16 rows (activations or weights).
hipError_t launch_quantize(const void* x_f16, int64_t rows, int64_t K, int32_t g,
                           void* q_u8, float* s, hipStream_t stream);

// Rows of the debug group sums: output row m goes to row (m - row0) / step of
// psum when that is a whole number below count; row0 = 0, step = 1, count = M
// keeps every row.  psum is then int32 [count, N, G].
struct PsumRows {
    int32_t row0 = 0;
    int32_t step = 1;
    int32_t count = 0;
};

// The address of the debug sum of (m, n, group j), or null for rows that are
// not kept.
__device__ inline int32_t* psum_at(int32_t* psum, const PsumRows& pr, int m, int n, int N, int G, int j)
{
    const int d = m - pr.row0;
    if (d < 0) return nullptr;
    const int q = d / pr.step;
    if (q * pr.step != d || q >= pr.count) return nullptr;
    return psum + ((int64_t)q * N + n) * G + j;
}

struct GemmProblem {
    const uint8_t* qa;
    const float* sa;
    const uint8_t* qw;
    const float* sw;
    int32_t M, N, K;
    int32_t ga, gw;       // group sizes along K of the two operands
    void* y16;            // fp16 [M, N]
    float* y32;           // fp32 [M, N] or null
    int32_t* psum;        // int32 [prows.count, N, K/min(ga,gw)] or null
    PsumRows prows;       // which output rows psum keeps
    void* ws;             // device workspace (gemm_workspace_bytes) or null
    size_t ws_bytes;
};

// The ping-pong kernel's K split of a partial last round of tiles: the last
// `tail` tiles (0: no split) run as `nparts` parts of K into an fp32
// workspace of `bytes`, then a reduction writes their Y.
struct PingpongSplit {
    int tiles = 0;
    int tail = 0;
    int nparts = 1;
    size_t bytes = 0;
    float* part = nullptr;
};
PingpongSplit pingpong_split(const GemmProblem& p);

// The K-outer kernel's K split (2 parts, or 1: none) and its fp32 workspace.
int kouter_kparts(const GemmProblem& p);
size_t kouter_workspace_bytes(const GemmProblem& p);

// The kernel launch_gemm runs for a shape (shapes and groups only): the
// weight-streaming kernels for few rows (row-streaming dot8, LDS-streaming
// MFMA, its K-outer variant, skinny MFMA), the tiled ones otherwise.
enum class GemmKernel { Gemv, Stream, Kouter, Skinny, Pingpong, Tiled };
GemmKernel gemm_kernel(const GemmProblem& p);

// Device workspace the call needs (0 for most shapes): the kernel choice of
// launch_gemm, shapes only.
size_t gemm_workspace_bytes(const GemmProblem& p);

// Picks the kernel for the shape: the row-streaming dot8 kernel (M <= 2), the
// LDS-streaming MFMA kernels (M <= 16, and 17..64 with K outside the column
// blocks), the skinny MFMA kernel (M <= 64, the group modes those two lack;
// these four stream the weights, groups >= 128), the ping-pong tiled kernel
// (groups of 128 or one group over K) or the tiled kernel (everything else).
hipError_t launch_gemm(const GemmProblem& p, hipStream_t stream);

hipError_t launch_gemm_tiled(const GemmProblem& p, hipStream_t stream);

// apex4_gemm_w4a4 / apex4_gemm_w4a4_debug after their own checks: every
// documented host-side check of the GEMM, then launch_gemm on `stream`.
// Returns an apex4_status code.
int32_t gemm_checked(const void* qa_u8, const float* s_a, int32_t group_a, const void* qw_u8, const float* s_w,
                     int32_t group_w, int64_t M, int64_t N, int64_t K, void* y_f16, float* y_f32, int64_t p_row0,
                     int64_t p_step, int64_t p_rows, int32_t* psum_dbg, void* workspace, size_t workspace_bytes,
                     void* stream);
bool pingpong_supports(const GemmProblem& p);
hipError_t launch_gemm_pingpong(const GemmProblem& p, hipStream_t stream);
// FP8-coded operands (apex4_gemm_w4a4_f8): qa, qw hold one E4M3 byte per code
hipError_t launch_gemm_pingpong_f8(const GemmProblem& p, hipStream_t stream);
// FP6-coded operands (apex4_gemm_w4a4_f6): qa, qw hold one 6-bit E2M3 field
// per code, packed in K order ([rows, 3K/4] bytes); groups of 128
bool f6_supports(const GemmProblem& p);
hipError_t launch_gemm_f6(const GemmProblem& p, hipStream_t stream);
hipError_t launch_quantize_f6(const void* x_f16, int64_t rows, int64_t K, void* q6, float* s, hipStream_t stream);
hipError_t launch_quantize_f8(const void* x_f16, int64_t rows, int64_t K, int group, void* q8, float* s,
                              hipStream_t stream);
bool gemv_supports(const GemmProblem& p);
hipError_t launch_gemm_gemv(const GemmProblem& p, hipStream_t stream);
// the row-streaming kernel quantizing its (1 or 2) fp16 activation rows itself
bool gemv_fused_supports(const GemmProblem& p);
hipError_t launch_gemm_gemv_fused(const GemmProblem& p, const void* x_f16, hipStream_t stream);
bool stream_supports(const GemmProblem& p);
hipError_t launch_gemm_stream(const GemmProblem& p, hipStream_t stream);
bool kouter_supports(const GemmProblem& p);
hipError_t launch_gemm_kouter(const GemmProblem& p, hipStream_t stream);
bool skinny_supports(const GemmProblem& p);
hipError_t launch_gemm_skinny(const GemmProblem& p, hipStream_t stream);

}  // namespace apex4
