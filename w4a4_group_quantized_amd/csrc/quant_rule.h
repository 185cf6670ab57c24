// The quantization rule on the GPU, shared by the quantization kernels and the
// decode kernel that quantizes its activation rows itself: symmetric INT4
// per group, scale = absmax / 7 (IEEE fp32 division), code = the
// round-to-nearest-even integer of the correctly rounded quotient x / scale,
// clamped to [-8, 7] (the APEX4 page's pure W4A4 scheme, with the readings of
// include/apex4.h).  Device functions only.
#ifndef APEX4_QUANT_RULE_H
#define APEX4_QUANT_RULE_H

#include <hip/hip_runtime.h>

#include <cstdint>

namespace apex4 {
namespace qrule {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));

__device__ inline float absmax8(const half8& h)
{
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf((float)h[i]));
    return m;
}

// 8 codes of one group-scale, packed little-nibble-first into one word.
//
// The rule rounds the correctly rounded fp32 quotient x / s.  Dividing per
// value costs ~10 instructions, so the quotient is taken as y = x * r with
// r = 1/s (correctly rounded, once per group): |y - fl(x/s)| <= 3 * 2^-24 *
// |x/s| < 1.5e-6 because |x/s| < 8, so y and fl(x/s) round to the same
// integer unless y lies within that distance of a half-integer; a chunk with
// such a value (a few in a million) is redone with the exact division.
__device__ inline uint32_t quantize8(const half8& h, float scale, bool nonzero)
{
    uint32_t word = 0;
    if (nonzero) {
        const float r = 1.0f / scale;
        float q[8];
        bool near_tie = false;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float y = (float)h[i] * r;
            q[i] = rintf(y);
            near_tie |= fabsf(y - q[i]) > 0.5f - 4e-6f;
        }
        if (near_tie) {
            // (rare) the whole chunk by the exact division
#pragma unroll
            for (int i = 0; i < 8; ++i) q[i] = rintf((float)h[i] / scale);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float c = fminf(fmaxf(q[i], -8.0f), 7.0f);
            word |= ((uint32_t)(int)c & 0xFu) << (4 * i);
        }
    }
    return word;
}

// max over aligned groups of N lanes (N = 4, 8, 16, 32) with DPP lane moves
// (no LDS round trip): quad swaps, then half-row and row mirrors; 32 lanes add
// one cross-row exchange
template <int CTRL>
__device__ inline float dpp_move(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

template <int N>
__device__ inline float group_max(float v)
{
    v = fmaxf(v, dpp_move<0xB1>(v));                      // quad_perm [1,0,3,2]: lane i <-> i ^ 1
    v = fmaxf(v, dpp_move<0x4E>(v));                      // quad_perm [2,3,0,1]: lane i <-> i ^ 2
    if (N >= 8) v = fmaxf(v, dpp_move<0x141>(v));         // row_half_mirror: i <-> 7 - i within 8
    if (N >= 16) v = fmaxf(v, dpp_move<0x140>(v));        // row_mirror: i <-> 15 - i within 16
    if (N >= 32) v = fmaxf(v, __shfl_xor(v, 16));
    return v;
}

}  // namespace qrule
}  // namespace apex4

#endif
