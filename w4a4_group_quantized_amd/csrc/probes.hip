// Measurement probes (include/apex4_probe.h): the int8 and FP6 matrix-unit
// rates, the HBM read rate, the fp32 vector-ALU rate and the LDS read rate of the GPU at
// hand, the ceilings the GEMM kernels are quoted against besides the datasheet
// peaks.
#include "apex4_probe.h"

#include <hip/hip_runtime.h>

namespace apex4 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int PROBE_BLOCKS = 1024;
constexpr int PROBE_THREADS = 256;

// 4 independent accumulators per wave, so that consecutive MFMAs never wait
// on each other; the operands are lane-dependent values the compiler cannot
// fold.
__global__ __launch_bounds__(PROBE_THREADS) void probe_mfma_kernel(int64_t iters, int32_t* sink)
{
    const int l = threadIdx.x;
    const v4i a = v4i{l, 3 * l + 1, 5 * l + 2, 7 * l + 3};
    const v4i b = v4i{11 * l + 5, 13 * l + 7, 17 * l + 9, 19 * l + 11};
    v16i c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int64_t i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, a, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, b, c3, 0, 0, 0);
    }
    int s = 0;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c0[r] ^ c1[r] ^ c2[r] ^ c3[r];
    if (s == 0x7fffffff) sink[0] = s;
}

// The same with v_mfma_scale_f32_32x32x64_f8f6f4 on FP6 E2M3 operands
// (format code 2 for both) and unit block scales (E8M0 127): the instruction
// of the FP6-coded GEMM.  The operand registers hold lane-dependent bits; six
// of the eight registers carry the 64 six-bit fields of a lane's row slice.
__global__ __launch_bounds__(PROBE_THREADS) void probe_mfma_f6_kernel(int64_t iters, int32_t* sink)
{
    const int l = threadIdx.x;
    const v8i a = v8i{l, 3 * l + 1, 5 * l + 2, 7 * l + 3, 9 * l + 4, 11 * l + 5, 0, 0};
    const v8i b = v8i{13 * l + 7, 17 * l + 9, 19 * l + 11, 23 * l + 13, 29 * l + 15, 31 * l + 17, 0, 0};
    v16f c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int64_t i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c0, 2, 2, 0, 127, 0, 127);
        c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c1, 2, 2, 0, 127, 0, 127);
        c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, a, c2, 2, 2, 0, 127, 0, 127);
        c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, b, c3, 2, 2, 0, 127, 0, 127);
    }
    float s = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
    if (s == 1234.5f) sink[0] = 1;
}

// Every wave reads whole 4 KB rows: lane l takes bytes [64 l, 64 l + 64) of a
// row as four 16-byte loads, rows dealt round-robin to the waves.
__global__ __launch_bounds__(PROBE_THREADS) void probe_read_kernel(const uint4* __restrict__ buf, int64_t rows,
                                                                   int32_t* sink)
{
    const int lane = threadIdx.x & 63;
    const int64_t gw = (int64_t)blockIdx.x * (PROBE_THREADS / 64) + (threadIdx.x >> 6);
    const int64_t nw = (int64_t)gridDim.x * (PROBE_THREADS / 64);
    uint32_t acc = 0;
    for (int64_t row = gw; row < rows; row += nw) {
        const uint4* p = buf + row * 256 + 4 * lane;
        const uint4 v0 = p[0], v1 = p[1], v2 = p[2], v3 = p[3];
        acc ^= v0.x ^ v1.y ^ v2.z ^ v3.w;
        acc += v0.w ^ v1.x ^ v2.y ^ v3.z;
    }
    if (acc == 0x7fffffffu) sink[0] = (int32_t)acc;
}

// 8 independent FMA chains per thread.
__global__ __launch_bounds__(PROBE_THREADS) void probe_valu_kernel(int64_t iters, float* sink)
{
    const float t = (float)threadIdx.x * 1e-3f;
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = t + (float)j;
    const float m = 0.9999f, c = 1e-4f;
    for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = fmaf(x[j], m, c);
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += x[j];
    if (s == -12345.0f) sink[0] = s;
}

// 16-byte LDS reads: every wave reads 1 KB contiguous pieces (lane l at 16 l:
// no bank conflicts) of a 16 KB buffer, 8 reads per iteration issued
// together and waited for in the same asm statement (so none can be hoisted
// out of the loop and no result is used before it has arrived); 16 waves per
// compute unit keep many reads in flight.
constexpr int LDS_PROBE_BYTES = 16384;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(PROBE_THREADS) void probe_lds_kernel(int64_t iters, int32_t* sink)
{
    __shared__ uint4 buf[LDS_PROBE_BYTES / 16];
    const int t = threadIdx.x, lane = t & 63;
    for (int i = t; i < LDS_PROBE_BYTES / 16; i += PROBE_THREADS)
        buf[i] = make_uint4(i, 3 * i + 1, 5 * i + 2, 7 * i + 3);
    __syncthreads();
    // byte address of this lane's 16 bytes in piece 0; the 8 reads take
    // pieces 0..7 (or 8..15 on odd iterations) at immediate offsets
    const uint32_t base = (uint32_t)(uintptr_t)buf + 16u * lane;
    u32x4 acc = {0, 0, 0, 0};
    for (int64_t i = 0; i < iters; ++i) {
        const uint32_t a = base + (((uint32_t)i & 1u) << 13);
        u32x4 v0, v1, v2, v3, v4, v5, v6, v7;
        asm volatile(
            "ds_read_b128 %0, %8\n"
            "ds_read_b128 %1, %8 offset:1024\n"
            "ds_read_b128 %2, %8 offset:2048\n"
            "ds_read_b128 %3, %8 offset:3072\n"
            "ds_read_b128 %4, %8 offset:4096\n"
            "ds_read_b128 %5, %8 offset:5120\n"
            "ds_read_b128 %6, %8 offset:6144\n"
            "ds_read_b128 %7, %8 offset:7168\n"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(v0), "=&v"(v1), "=&v"(v2), "=&v"(v3), "=&v"(v4), "=&v"(v5), "=&v"(v6), "=&v"(v7)
            : "v"(a)
            : "memory");
        acc ^= v0 ^ v1 ^ v2 ^ v3;
        acc += v4 ^ v5 ^ v6 ^ v7;
    }
    const uint32_t s = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (s == 0x7fffffffu) sink[0] = (int32_t)s;
}

apex4_status launched()
{
    return hipGetLastError() == hipSuccess ? APEX4_OK : APEX4_ERR_HIP;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

}  // namespace
}  // namespace apex4

extern "C" {

apex4_status apex4_probe_mfma_i8(int64_t iters, int32_t* sink, double* ops_out, void* stream)
{
    using namespace apex4;
    if (iters < 1 || sink == nullptr || ops_out == nullptr) return APEX4_ERR_INVALID_ARG;
    if (!aligned(sink, 4)) return APEX4_ERR_ALIGNMENT;
    *ops_out = (double)PROBE_BLOCKS * (PROBE_THREADS / 64) * (double)iters * 4 * 2 * 32.0 * 32 * 32;
    probe_mfma_kernel<<<PROBE_BLOCKS, PROBE_THREADS, 0, (hipStream_t)stream>>>(iters, sink);
    return launched();
}

apex4_status apex4_probe_mfma_f6(int64_t iters, int32_t* sink, double* ops_out, void* stream)
{
    using namespace apex4;
    if (iters < 1 || sink == nullptr || ops_out == nullptr) return APEX4_ERR_INVALID_ARG;
    if (!aligned(sink, 4)) return APEX4_ERR_ALIGNMENT;
    *ops_out = (double)PROBE_BLOCKS * (PROBE_THREADS / 64) * (double)iters * 4 * 2 * 32.0 * 32 * 64;
    probe_mfma_f6_kernel<<<PROBE_BLOCKS, PROBE_THREADS, 0, (hipStream_t)stream>>>(iters, sink);
    return launched();
}

apex4_status apex4_probe_hbm_read(const void* buf, int64_t bytes, int32_t* sink, double* bytes_out, void* stream)
{
    using namespace apex4;
    if (buf == nullptr || sink == nullptr || bytes_out == nullptr || bytes <= 0 || bytes % 4096 != 0)
        return APEX4_ERR_INVALID_ARG;
    if (!aligned(buf, 16) || !aligned(sink, 4)) return APEX4_ERR_ALIGNMENT;
    *bytes_out = (double)bytes;
    probe_read_kernel<<<PROBE_BLOCKS, PROBE_THREADS, 0, (hipStream_t)stream>>>(static_cast<const uint4*>(buf),
                                                                               bytes / 4096, sink);
    return launched();
}

apex4_status apex4_probe_valu_f32(int64_t iters, float* sink, double* flops_out, void* stream)
{
    using namespace apex4;
    if (iters < 1 || sink == nullptr || flops_out == nullptr) return APEX4_ERR_INVALID_ARG;
    if (!aligned(sink, 4)) return APEX4_ERR_ALIGNMENT;
    *flops_out = (double)PROBE_BLOCKS * PROBE_THREADS * (double)iters * 8 * 2;
    probe_valu_kernel<<<PROBE_BLOCKS, PROBE_THREADS, 0, (hipStream_t)stream>>>(iters, sink);
    return launched();
}

apex4_status apex4_probe_lds_read(int64_t iters, int32_t* sink, double* bytes_out, void* stream)
{
    using namespace apex4;
    if (iters < 1 || iters > (int64_t(1) << 30) || sink == nullptr || bytes_out == nullptr)
        return APEX4_ERR_INVALID_ARG;
    if (!aligned(sink, 4)) return APEX4_ERR_ALIGNMENT;
    *bytes_out = (double)PROBE_BLOCKS * PROBE_THREADS * (double)iters * 8 * 16;
    probe_lds_kernel<<<PROBE_BLOCKS, PROBE_THREADS, 0, (hipStream_t)stream>>>(iters, sink);
    return launched();
}

}  // extern "C"
