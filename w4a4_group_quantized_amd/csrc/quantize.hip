// Symmetric per-group INT4 quantization on gfx950 (activations online, weights
// offline): the rule of the APEX4 page's pure W4A4 scheme, with the readings
// spelled out in include/apex4.h.  Memory-bound: 16-byte fp16 loads, one
// packed 32-bit word (8 codes) per thread, group absmax by cross-lane
// butterflies (or the codes as FP8 bytes, for the FP8-operand GEMM).  The
// scale and every quotient are IEEE fp32 divisions (the
// library is built with correctly rounded fp32 division) and the rounding is
// v_rndne_f32, so the codes are bit-identical to the rule (quant_rule.h).
#include "internal.h"
#include "quant_rule.h"

namespace apex4 {
namespace {

using namespace qrule;

// The same 8 codes as FP8 E4M3 values, one byte each in K order (the codes
// -8..7 are exact in E4M3; -0 is stored as +0).
__device__ inline uint2 quantize8_f8(const half8& h, float scale, bool nonzero)
{
    float c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = 0.0f;
    if (nonzero) {
        const uint32_t word = quantize8(h, scale, true);
#pragma unroll
        for (int i = 0; i < 8; ++i) c[i] = (float)((int)(word << (28 - 4 * i)) >> 28) + 0.0f;
    }
    uint32_t lo = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], lo, true);
    uint32_t hi = __builtin_amdgcn_cvt_pk_fp8_f32(c[4], c[5], 0, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(c[6], c[7], hi, true);
    return make_uint2(lo, hi);
}

// Group sizes 32..256: a group is G/8 consecutive lanes of one wave.  F8:
// the codes as FP8 bytes ([rows, K]) instead of packed nibbles.
template <int G, bool F8>
__global__ __launch_bounds__(256) void quantize_groups_kernel(const half8* __restrict__ x,
                                                              int64_t n8,
                                                              void* __restrict__ q,
                                                              float* __restrict__ s)
{
    constexpr int TPG = G / 8;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const bool live = t < n8;
    half8 h = {};
    if (live) h = x[t];
    const float amax = group_max<TPG>(absmax8(h));
    const float scale = amax / 7.0f;
    const bool nz = amax != 0.0f;
    if (live) {
        if (F8) static_cast<uint2*>(q)[t] = quantize8_f8(h, scale, nz);
        else static_cast<uint32_t*>(q)[t] = quantize8(h, scale, nz);
        if ((t % TPG) == 0) s[t / TPG] = nz ? scale : 0.0f;
    }
}

// FP6-coded operands.  A code c is the 6-bit E2M3 field (c < 0) << 5 | |c|:
// with a 3-bit mantissa and exponent bias 1, the magnitudes 0..15 of that
// field are the subnormal and first-binade values 0/8 .. 15/8, so the field
// holds c / 8 exactly (-8 included; -0 is stored as +0).  The 128 fields of a
// (row, group) pack little-endian into 96 bytes, code k of the group at bits
// 6k .. 6k+5; those 96 bytes are six 16-byte chunks.  Tiled layout: rows in
// blocks of 64 (the last block padded with zero rows); tile (row block b,
// group j) is 6 KB at byte ((b * G + j) * 6) * 1024, chunk q of row i of the
// block at + q * 1024 + i * 16.  A tile's chunk q of 64 rows is then one
// contiguous KB: one direct-to-LDS load of the GEMM.
//
// One thread per (row, group): 128 codes (sixteen 16-byte loads), 96 bytes
// out.  The 64 lanes of a wave are the 64 rows of one block and group, so
// each of the thread's six chunk stores is one contiguous KB of the tile.
__device__ inline uint32_t f6_field(uint32_t word, int i)
{
    const int c = (int)(word << (28 - 4 * i)) >> 28;
    return (c < 0 ? 32u : 0u) | (uint32_t)(c < 0 ? -c : c);
}

__global__ __launch_bounds__(256) void quantize_f6_kernel(const half8* __restrict__ x, int64_t rows, int64_t K,
                                                          int64_t n_threads, uint4* __restrict__ q,
                                                          float* __restrict__ s)
{
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t G = K / 128;
    const int64_t rest = t >> 6, j = rest % G, rb = rest / G;
    const int64_t r = rb * 64 + (t & 63);
    const bool in = t < n_threads;
    const bool live = in && r < rows;              // padding rows of the last block: zeros
    half8 h[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) h[i] = half8{};
    if (live) {
        const half8* xr = x + r * (K / 8) + 16 * j;
#pragma unroll
        for (int i = 0; i < 16; ++i) h[i] = xr[i];
    }
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) m = fmaxf(m, absmax8(h[i]));
    const float scale = m / 7.0f;
    const bool nz = m != 0.0f;
    if (in) {
        uint32_t o[24];
#pragma unroll
        for (int i = 0; i < 24; ++i) o[i] = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t w = quantize8(h[i], scale, nz && live);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const uint32_t f = f6_field(w, k);
                const int b = 6 * (8 * i + k);     // bit position in the 96 bytes
                o[b / 32] |= f << (b % 32);
                if (b % 32 > 26) o[b / 32 + 1] |= f >> (32 - b % 32);
            }
        }
        uint4* tile = q + (rb * G + j) * 6 * 64 + (t & 63);
#pragma unroll
        for (int c = 0; c < 6; ++c) tile[c * 64] = make_uint4(o[4 * c], o[4 * c + 1], o[4 * c + 2], o[4 * c + 3]);
        if (live) s[r * G + j] = nz ? scale : 0.0f;
    }
}

// One group per row (per-channel scales, any K % 8 == 0): one block per row.
__global__ __launch_bounds__(256) void quantize_rows_kernel(const half8* __restrict__ x,
                                                            int64_t k8,
                                                            uint32_t* __restrict__ q,
                                                            float* __restrict__ s)
{
    __shared__ float part[4];
    const int64_t row = blockIdx.x;
    const half8* xr = x + row * k8;
    float amax = 0.0f;
    for (int64_t i = threadIdx.x; i < k8; i += 256) amax = fmaxf(amax, absmax8(xr[i]));
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
    const float scale = amax / 7.0f;
    const bool nz = amax != 0.0f;
    uint32_t* qr = q + row * k8;
    for (int64_t i = threadIdx.x; i < k8; i += 256) qr[i] = quantize8(xr[i], scale, nz);
    if (threadIdx.x == 0) s[row] = nz ? scale : 0.0f;
}

}  // namespace

hipError_t launch_quantize(const void* x_f16, int64_t rows, int64_t K, int32_t g, void* q_u8,
                           float* s, hipStream_t stream)
{
    const half8* x = static_cast<const half8*>(x_f16);
    uint32_t* q = static_cast<uint32_t*>(q_u8);
    const int64_t n8 = rows * (K / 8);
    const unsigned blocks = (unsigned)((n8 + 255) / 256);
    switch (g) {
    case 32: quantize_groups_kernel<32, false><<<blocks, 256, 0, stream>>>(x, n8, q, s); break;
    case 64: quantize_groups_kernel<64, false><<<blocks, 256, 0, stream>>>(x, n8, q, s); break;
    case 128: quantize_groups_kernel<128, false><<<blocks, 256, 0, stream>>>(x, n8, q, s); break;
    case 256: quantize_groups_kernel<256, false><<<blocks, 256, 0, stream>>>(x, n8, q, s); break;
    default:  // g == K, checked by the caller
        quantize_rows_kernel<<<(unsigned)rows, 256, 0, stream>>>(x, K / 8, q, s);
        break;
    }
    return hipGetLastError();
}

hipError_t launch_quantize_f8(const void* x_f16, int64_t rows, int64_t K, int group, void* q8, float* s,
                              hipStream_t stream)
{
    // group: 64 or 128, checked by the caller
    const int64_t n8 = rows * (K / 8);
    const unsigned blocks = (unsigned)((n8 + 255) / 256);
    const half8* x = static_cast<const half8*>(x_f16);
    if (group == 64) quantize_groups_kernel<64, true><<<blocks, 256, 0, stream>>>(x, n8, q8, s);
    else quantize_groups_kernel<128, true><<<blocks, 256, 0, stream>>>(x, n8, q8, s);
    return hipGetLastError();
}

}  // namespace apex4

namespace apex4 {

hipError_t launch_quantize_f6(const void* x_f16, int64_t rows, int64_t K, void* q6, float* s, hipStream_t stream)
{
    // rows padded to whole blocks of 64
    const int64_t n_threads = (rows + 63) / 64 * 64 * (K / 128);
    const unsigned blocks = (unsigned)((n_threads + 255) / 256);
    quantize_f6_kernel<<<blocks, 256, 0, stream>>>(static_cast<const half8*>(x_f16), rows, K, n_threads,
                                                   static_cast<uint4*>(q6), s);
    return hipGetLastError();
}

}  // namespace apex4
