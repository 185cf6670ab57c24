// C ABI of libapex4 (include/apex4.h): host-side argument checks, then the
// launch on the caller's stream.  Every check runs before any HIP call, so a
// rejected call touches neither the device nor the caller's memory.
#include "apex4.h"

#include <cstdint>

#include "internal.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool small_group(int64_t g) { return g == 32 || g == 64 || g == 128 || g == 256; }

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;

apex4_status check_quantize(const void* x, int64_t rows, int64_t K, int32_t g, const void* q,
                            const float* s)
{
    if (rows < 0 || rows > kMaxDim || K <= 0 || K > kMaxDim || K % 8 != 0)
        return APEX4_ERR_INVALID_ARG;
    if (g <= 0 || K % g != 0) return APEX4_ERR_INVALID_ARG;
    if (!small_group(g) && g != K) return APEX4_ERR_UNSUPPORTED;
    if (rows == 0) return APEX4_OK;
    if (!x || !q || !s) return APEX4_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(q, 4) || !aligned(s, 4)) return APEX4_ERR_ALIGNMENT;
    return APEX4_OK;
}

apex4_status to_status(hipError_t e) { return e == hipSuccess ? APEX4_OK : APEX4_ERR_HIP; }

// One group over all of K keeps the kernels' int32 group sum (of the codes
// widened to 16 c, i.e. 256 times the sum) over the whole row: |256 P| <=
// 256 * 64 * K must stay below 2^31, so K < 2^17 there.
constexpr int64_t kMaxPerChannelK = int64_t(1) << 17;

bool per_channel_overflows(int64_t K, int32_t group_a, int32_t group_w)
{
    return group_a == K && group_w == K && K >= kMaxPerChannelK;
}


}  // namespace

extern "C" {

const char* apex4_status_string(apex4_status s)
{
    switch (s) {
    case APEX4_OK: return "ok";
    case APEX4_ERR_INVALID_ARG: return "invalid argument";
    case APEX4_ERR_UNSUPPORTED: return "unsupported group-size combination";
    case APEX4_ERR_ALIGNMENT: return "misaligned pointer";
    case APEX4_ERR_WORKSPACE: return "workspace too small";
    case APEX4_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

apex4_status apex4_quantize_act(const void* x_f16, int64_t M, int64_t K, int32_t group_a,
                                void* qa_u8, float* s_a, void* stream)
{
    const apex4_status st = check_quantize(x_f16, M, K, group_a, qa_u8, s_a);
    if (st != APEX4_OK || M == 0) return st;
    return to_status(apex4::launch_quantize(x_f16, M, K, group_a, qa_u8, s_a,
                                            static_cast<hipStream_t>(stream)));
}

apex4_status apex4_pack_weight(const void* w_f16, int64_t N, int64_t K, int32_t group_w,
                               void* qw_u8, float* s_w, void* stream)
{
    const apex4_status st = check_quantize(w_f16, N, K, group_w, qw_u8, s_w);
    if (st != APEX4_OK || N == 0) return st;
    return to_status(apex4::launch_quantize(w_f16, N, K, group_w, qw_u8, s_w,
                                            static_cast<hipStream_t>(stream)));
}

namespace {

size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

// the GEMM problem of a linear call (shape and groups only), or false
bool linear_problem(int64_t M, int64_t N, int64_t K, int32_t group_a, int32_t group_w, apex4::GemmProblem& p)
{
    if (M <= 0 || N <= 0 || M > kMaxDim || N > kMaxDim || K <= 0 || K > kMaxDim || K % 128 != 0) return false;
    if (group_a <= 0 || group_w <= 0 || K % group_a != 0 || K % group_w != 0) return false;
    if (per_channel_overflows(K, group_a, group_w)) return false;
    p = apex4::GemmProblem{};
    p.M = static_cast<int32_t>(M);
    p.N = static_cast<int32_t>(N);
    p.K = static_cast<int32_t>(K);
    p.ga = group_a;
    p.gw = group_w;
    return true;
}

}  // namespace

size_t apex4_linear_workspace_size(int64_t M, int64_t N, int64_t K, int32_t group_a, int32_t group_w)
{
    apex4::GemmProblem p;
    if (!linear_problem(M, N, K, group_a, group_w, p)) return 0;
    if (apex4::gemv_fused_supports(p)) return 0;
    return align256((size_t)M * (K / 2)) + align256((size_t)M * (K / group_a) * 4) + apex4::gemm_workspace_bytes(p);
}

apex4_status apex4_linear_w4a4(const void* x_f16, int32_t group_a, const void* qw_u8, const float* s_w,
                               int32_t group_w, int64_t M, int64_t N, int64_t K, void* y_f16, float* y_f32,
                               void* workspace, size_t workspace_bytes, void* stream)
{
    // the checks of apex4_quantize_act and apex4_gemm_w4a4
    if (M < 0 || N < 0 || M > kMaxDim || N > kMaxDim || K <= 0 || K > kMaxDim || K % 128 != 0)
        return APEX4_ERR_INVALID_ARG;
    if (group_a <= 0 || group_w <= 0 || K % group_a != 0 || K % group_w != 0) return APEX4_ERR_INVALID_ARG;
    if (!small_group(group_a) && group_a != K) return APEX4_ERR_UNSUPPORTED;
    if (!(group_w == group_a || group_w == K)) return APEX4_ERR_UNSUPPORTED;
    if (per_channel_overflows(K, group_a, group_w)) return APEX4_ERR_UNSUPPORTED;
    const size_t need = apex4_linear_workspace_size(M, N, K, group_a, group_w);
    if (workspace_bytes < need || (need > 0 && !workspace)) return APEX4_ERR_WORKSPACE;
    if (M == 0 || N == 0) return APEX4_OK;
    if (!x_f16 || !qw_u8 || !s_w || !y_f16) return APEX4_ERR_INVALID_ARG;
    if (!aligned(x_f16, 16) || !aligned(qw_u8, 16) || !aligned(s_w, 4) || !aligned(y_f16, 2) ||
        !aligned(y_f32, 4) || !aligned(workspace, 256))
        return APEX4_ERR_ALIGNMENT;
    apex4::GemmProblem p;
    linear_problem(M, N, K, group_a, group_w, p);
    p.qw = static_cast<const uint8_t*>(qw_u8);
    p.sw = s_w;
    p.y16 = y_f16;
    p.y32 = y_f32;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (apex4::gemv_fused_supports(p)) return to_status(apex4::launch_gemm_gemv_fused(p, x_f16, st));
    // quantize into the workspace, then the GEMM (its own workspace after)
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    const size_t qa_bytes = align256((size_t)M * (K / 2)), sa_bytes = align256((size_t)M * (K / group_a) * 4);
    uint8_t* qa = ws;
    float* sa = reinterpret_cast<float*>(ws + qa_bytes);
    hipError_t e = apex4::launch_quantize(x_f16, M, K, group_a, qa, sa, st);
    if (e != hipSuccess) return APEX4_ERR_HIP;
    p.qa = qa;
    p.sa = sa;
    p.ws = ws + qa_bytes + sa_bytes;
    p.ws_bytes = workspace_bytes - qa_bytes - sa_bytes;
    return to_status(apex4::launch_gemm(p, st));
}

apex4_status apex4_quantize_f8(const void* x_f16, int64_t rows, int64_t K, int32_t group, void* q8,
                               float* s, void* stream)
{
    if (group != 128 && group != 64)
        return group > 0 && K > 0 && K % group == 0 ? APEX4_ERR_UNSUPPORTED : APEX4_ERR_INVALID_ARG;
    const apex4_status st = check_quantize(x_f16, rows, K, group, q8, s);
    if (st != APEX4_OK || rows == 0) return st;
    if (!aligned(q8, 8)) return APEX4_ERR_ALIGNMENT;
    return to_status(apex4::launch_quantize_f8(x_f16, rows, K, group, q8, s, static_cast<hipStream_t>(stream)));
}

apex4_status apex4_gemm_w4a4_f8(const void* qa8, const float* s_a, const void* qw8, const float* s_w,
                                int32_t group, int64_t M, int64_t N, int64_t K, void* y_f16, float* y_f32,
                                int32_t* psum_dbg, void* stream)
{
    if (M < 0 || N < 0 || M > kMaxDim || N > kMaxDim || K <= 0 || K > kMaxDim || K % 128 != 0)
        return APEX4_ERR_INVALID_ARG;
    if (group <= 0 || K % group != 0) return APEX4_ERR_INVALID_ARG;
    if (group != 128 && group != 64) return APEX4_ERR_UNSUPPORTED;
    if (psum_dbg && (unsigned __int128)M * (uint64_t)N * (uint64_t)(K / group) > (uint64_t)kMaxDim)
        return APEX4_ERR_INVALID_ARG;
    // 32-bit offsets within a 256-row block of operand bytes
    if ((uint64_t)K * 256 >= (1ull << 31)) return APEX4_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return APEX4_OK;
    if (!qa8 || !s_a || !qw8 || !s_w || !y_f16) return APEX4_ERR_INVALID_ARG;
    if (!aligned(qa8, 16) || !aligned(qw8, 16) || !aligned(s_a, 4) || !aligned(s_w, 4) || !aligned(y_f16, 2) ||
        !aligned(y_f32, 4) || !aligned(psum_dbg, 4))
        return APEX4_ERR_ALIGNMENT;
    apex4::GemmProblem p{};
    p.qa = static_cast<const uint8_t*>(qa8);
    p.sa = s_a;
    p.qw = static_cast<const uint8_t*>(qw8);
    p.sw = s_w;
    p.M = static_cast<int32_t>(M);
    p.N = static_cast<int32_t>(N);
    p.K = static_cast<int32_t>(K);
    p.ga = group;
    p.gw = group;
    p.y16 = y_f16;
    p.y32 = y_f32;
    p.psum = psum_dbg;
    p.prows.count = static_cast<int32_t>(M);
    return to_status(apex4::launch_gemm_pingpong_f8(p, static_cast<hipStream_t>(stream)));
}

apex4_status apex4_quantize_f6(const void* x_f16, int64_t rows, int64_t K, int32_t group, void* q6, float* s,
                               void* stream)
{
    if (group != 128) return group > 0 && K > 0 && K % group == 0 ? APEX4_ERR_UNSUPPORTED : APEX4_ERR_INVALID_ARG;
    const apex4_status st = check_quantize(x_f16, rows, K, group, q6, s);
    if (st != APEX4_OK || rows == 0) return st;
    if (!aligned(q6, 16)) return APEX4_ERR_ALIGNMENT;
    return to_status(apex4::launch_quantize_f6(x_f16, rows, K, q6, s, static_cast<hipStream_t>(stream)));
}

apex4_status apex4_gemm_w4a4_f6(const void* qa6, const float* s_a, const void* qw6, const float* s_w, int64_t M,
                                int64_t N, int64_t K, void* y_f16, float* y_f32, int32_t* psum_dbg,
                                void* workspace, size_t workspace_bytes, void* stream)
{
    if (M < 0 || N < 0 || M > kMaxDim || N > kMaxDim || K <= 0 || K > kMaxDim || K % 128 != 0)
        return APEX4_ERR_INVALID_ARG;
    if (psum_dbg && (unsigned __int128)M * (uint64_t)N * (uint64_t)(K / 128) > (uint64_t)kMaxDim)
        return APEX4_ERR_INVALID_ARG;
    apex4::GemmProblem p{};
    p.M = static_cast<int32_t>(M);
    p.N = static_cast<int32_t>(N);
    p.K = static_cast<int32_t>(K);
    p.ga = 128;
    p.gw = 128;
    // 32-bit offsets within a 256-row block of operand bytes
    if (!apex4::f6_supports(p)) return APEX4_ERR_UNSUPPORTED;
    const size_t need = apex4_gemm_workspace_size(M, N, K, 128, 128);
    if (workspace_bytes < need || (need > 0 && !workspace)) return APEX4_ERR_WORKSPACE;
    if (M == 0 || N == 0) return APEX4_OK;
    if (!qa6 || !s_a || !qw6 || !s_w || !y_f16) return APEX4_ERR_INVALID_ARG;
    if (!aligned(qa6, 16) || !aligned(qw6, 16) || !aligned(s_a, 4) || !aligned(s_w, 4) || !aligned(y_f16, 2) ||
        !aligned(y_f32, 4) || !aligned(psum_dbg, 4) || !aligned(workspace, 16))
        return APEX4_ERR_ALIGNMENT;
    p.qa = static_cast<const uint8_t*>(qa6);
    p.sa = s_a;
    p.qw = static_cast<const uint8_t*>(qw6);
    p.sw = s_w;
    p.y16 = y_f16;
    p.y32 = y_f32;
    p.psum = psum_dbg;
    p.prows.count = static_cast<int32_t>(M);
    p.ws = workspace;
    p.ws_bytes = workspace_bytes;
    return to_status(apex4::launch_gemm_f6(p, static_cast<hipStream_t>(stream)));
}

size_t apex4_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int32_t group_a, int32_t group_w)
{
    // shapes apex4_gemm_w4a4 rejects, or that launch nothing, need none
    if (M <= 0 || N <= 0 || M > kMaxDim || N > kMaxDim || K <= 0 || K > kMaxDim || K % 128 != 0) return 0;
    if (group_a <= 0 || group_w <= 0 || K % group_a != 0 || K % group_w != 0) return 0;
    if (per_channel_overflows(K, group_a, group_w)) return 0;
    apex4::GemmProblem p{};
    p.M = static_cast<int32_t>(M);
    p.N = static_cast<int32_t>(N);
    p.K = static_cast<int32_t>(K);
    p.ga = group_a;
    p.gw = group_w;
    return apex4::gemm_workspace_bytes(p);
}

apex4_status apex4_gemm_w4a4(const void* qa_u8, const float* s_a, int32_t group_a,
                             const void* qw_u8, const float* s_w, int32_t group_w, int64_t M,
                             int64_t N, int64_t K, void* y_f16, float* y_f32, int32_t* psum_dbg,
                             void* workspace, size_t workspace_bytes, void* stream)
{
    return apex4::gemm_checked(qa_u8, s_a, group_a, qw_u8, s_w, group_w, M, N, K, y_f16, y_f32, 0, 1, M, psum_dbg,
                        workspace, workspace_bytes, stream);
}

apex4_status apex4_gemm_w4a4_debug(const void* qa_u8, const float* s_a, int32_t group_a,
                                   const void* qw_u8, const float* s_w, int32_t group_w, int64_t M,
                                   int64_t N, int64_t K, void* y_f16, float* y_f32, int64_t p_row0,
                                   int64_t p_step, int64_t p_rows, int32_t* psum_dbg, void* workspace,
                                   size_t workspace_bytes, void* stream)
{
    if (p_row0 < 0 || p_step < 1 || p_rows < 0 || p_row0 > kMaxDim || p_step > kMaxDim || p_rows > kMaxDim)
        return APEX4_ERR_INVALID_ARG;
    // every kept row lies inside Y
    if (M > 0 && p_rows > 0 && p_row0 + (p_rows - 1) * p_step >= M) return APEX4_ERR_INVALID_ARG;
    if (p_rows > 0 && !psum_dbg) return APEX4_ERR_INVALID_ARG;
    return apex4::gemm_checked(qa_u8, s_a, group_a, qw_u8, s_w, group_w, M, N, K, y_f16, y_f32, p_row0, p_step, p_rows,
                        p_rows > 0 ? psum_dbg : nullptr, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace apex4 {

apex4_status gemm_checked(const void* qa_u8, const float* s_a, int32_t group_a, const void* qw_u8,
                          const float* s_w, int32_t group_w, int64_t M, int64_t N, int64_t K, void* y_f16,
                          float* y_f32, int64_t p_row0, int64_t p_step, int64_t p_rows, int32_t* psum_dbg,
                          void* workspace, size_t workspace_bytes, void* stream)
{
    if (M < 0 || N < 0 || M > kMaxDim || N > kMaxDim || K <= 0 || K > kMaxDim || K % 128 != 0)
        return APEX4_ERR_INVALID_ARG;
    if (group_a <= 0 || group_w <= 0 || K % group_a != 0 || K % group_w != 0)
        return APEX4_ERR_INVALID_ARG;
    if (!small_group(group_a) && group_a != K) return APEX4_ERR_UNSUPPORTED;
    if (!(group_w == group_a || group_w == K)) return APEX4_ERR_UNSUPPORTED;
    if (per_channel_overflows(K, group_a, group_w)) return APEX4_ERR_UNSUPPORTED;
    const int64_t gs = group_a < group_w ? group_a : group_w;
    if (psum_dbg && (unsigned __int128)p_rows * (uint64_t)N * (uint64_t)(K / gs) > (uint64_t)kMaxDim)
        return APEX4_ERR_INVALID_ARG;
    const size_t need = apex4_gemm_workspace_size(M, N, K, group_a, group_w);
    if (workspace_bytes < need || (need > 0 && !workspace)) return APEX4_ERR_WORKSPACE;
    if (M == 0 || N == 0) return APEX4_OK;
    if (!qa_u8 || !s_a || !qw_u8 || !s_w || !y_f16) return APEX4_ERR_INVALID_ARG;
    if (!aligned(qa_u8, 16) || !aligned(qw_u8, 16) || !aligned(s_a, 4) || !aligned(s_w, 4) ||
        !aligned(y_f16, 2) || !aligned(y_f32, 4) || !aligned(psum_dbg, 4) || !aligned(workspace, 16))
        return APEX4_ERR_ALIGNMENT;

    apex4::GemmProblem p{};
    p.qa = static_cast<const uint8_t*>(qa_u8);
    p.sa = s_a;
    p.qw = static_cast<const uint8_t*>(qw_u8);
    p.sw = s_w;
    p.M = static_cast<int32_t>(M);
    p.N = static_cast<int32_t>(N);
    p.K = static_cast<int32_t>(K);
    p.ga = group_a;
    p.gw = group_w;
    p.y16 = y_f16;
    p.y32 = y_f32;
    p.psum = psum_dbg;
    p.prows.row0 = static_cast<int32_t>(p_row0);
    p.prows.step = static_cast<int32_t>(p_step);
    p.prows.count = static_cast<int32_t>(p_rows);
    p.ws = workspace;
    p.ws_bytes = workspace_bytes;
    return to_status(apex4::launch_gemm(p, static_cast<hipStream_t>(stream)));
}

}  // namespace apex4

