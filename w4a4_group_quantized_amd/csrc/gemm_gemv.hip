// W4A4 GEMM for one or two token rows (decode; built for M <= 4) on gfx950: weight rows
// streamed whole by single waves, INT4 x INT4 products on v_dot8c_i32_i4.
//
// With a handful of tokens the product is bound by reading the packed weights
// once (the blog page "Why INT4 Weight-Only Quantization Doesn't Speed Up
// Prefill" works through this).  What matters is the access pattern: a wave
// that reads whole weight rows (4 x 16-byte loads per lane cover 4 KB of one
// row) streams a decode-sized matrix at ~6 TB/s on this chip, where reading
// 64-byte pieces of 32 rows at a time (the shape an MFMA operand wants)
// reaches ~3.7 TB/s.  So here each wave owns whole rows n of W, and the
// products need no matrix unit: v_dot8c_i32_i4 multiplies the 8 signed
// nibbles of a packed weight word with those of a packed activation word and
// adds them to an int32, exactly, in one vector instruction (the packed
// layout is the instruction's operand layout: no widening).
//
// Per row, lane l owns the 128-code units u = l, l+64, ... of the row (64
// packed bytes each, one group at g = 128).  For each activation row m the
// lane forms the exact group sum P = sum of 16 dot8 over the unit, then the
// rescale t = (s_a[m,j] * s_w[n,j]) * P in fp32 and adds it to its running
// sum (units in ascending order).  At the end of the row the 64 lane sums are
// added by a fixed butterfly and lane 0 writes Y[m, n].  Groups of 256 add the
// int32 sums of lane pairs before the rescale; one group over K adds all int32
// sums of the row first and rescales once; mixed mode (per-channel weight
// scales) rescales with s_a and applies s_w to the row sum.
//
// The activation rows and their scales are copied to LDS once per workgroup;
// their loads go out first and the first weight loads right after, so the
// wait for the copy leaves the weights in flight (issued the other way
// round, that wait also waited for the weights' HBM latency).  Per weight word the lane issues M dot8 and reads M activation
// words from LDS, so the kernel stays at the weight-streaming rate only for
// a few rows: from 3 rows on the LDS-streaming MFMA kernel is faster, and the
// dispatch sends only 1 or 2 rows here.  Lane l reads the four 16-byte quads
// of its unit starting at quad (l >> 1) & 3, for activations and weights
// alike, so that 8 consecutive lanes hit distinct LDS banks.
#include "internal.h"
#include "quant_rule.h"

namespace apex4 {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int UNIT = 128;                    // codes per lane unit
constexpr int UNIT_BYTES = UNIT / 2;         // 64 packed bytes = 4 quads of 16
constexpr int WAVES = 8;                     // waves per workgroup
constexpr int THREADS = WAVES * 64;
constexpr int PF = 2;                        // units of loads in flight ahead
constexpr uint32_t OOB = 0x80000000u;        // past every buffer: reads zeros

struct GemvArgs {
    const uint8_t* qa;
    const float* sa;
    const uint8_t* qw;
    const float* sw;
    int M, N, K;
    int Ga, Gw;        // scale columns per row: K/ga, K/gw
    int ga;            // activation group size
    int G;             // K / gs
    int U;             // units per row: K / 128
    int lds_qa;        // bytes of activation rows in LDS: M * K/2, 16-byte multiple
    const _Float16* x; // fused quantization: the fp16 activation rows [M, K]
    _Float16* y16;
    float* y32;
    int32_t* psum;
    PsumRows prows;
};

__device__ inline __amdgpu_buffer_rsrc_t buffer_of(const void* p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// fixed-order sum over the 64 lanes (the result is in every lane)
__device__ inline float wave_sum(float v)
{
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
    return v;
}

__device__ inline int wave_sum_int(int v)
{
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
    return v;
}

// MR: activation rows handled (M <= MR).  GM: 1 (groups of 128), 2 (groups of
// 256) or 0 (one group over K).  MIXED: per-channel weight scales with
// activation groups of 128.  FUSED: the workgroup quantizes the fp16
// activation rows itself (groups of 128 or 256), by the rule of the
// quantization kernels, into the LDS layout the copy would fill.
template <int MR, int GM, bool MIXED, bool DEBUG_P, bool FUSED = false>
__global__ __launch_bounds__(THREADS) void gemm_gemv_kernel(GemvArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int gwave = blockIdx.x * WAVES + wave, nwaves = gridDim.x * WAVES;
    const uint32_t rowbytes = (uint32_t)a.K / 2;
    const int passes = (a.U + 63) / 64;                 // units per lane per row
    const int rows_w = gwave < a.N ? (a.N - 1 - gwave) / nwaves + 1 : 0;
    const int items = rows_w * passes;                  // (row, pass) pairs of this wave
    const __amdgpu_buffer_rsrc_t rW = buffer_of(a.qw, (uint32_t)a.N * rowbytes);
    const __amdgpu_buffer_rsrc_t rS = buffer_of(a.sw, (uint32_t)a.N * a.Gw * 4);
    const int rot = (lane >> 1) & 3;                    // first quad of this lane

    // --- the weight stream of item i: unit u = lane + 64*pass of row n ---
    uint4 wq[PF][4];
    float ws[PF];
    auto issue = [&](int slot, int i) {
        const int r = i / passes, p = i - r * passes;
        const int n = gwave + nwaves * r;
        const int u = lane + 64 * p;
        const bool live = i < items && u < a.U;
        const uint32_t base = (uint32_t)n * rowbytes + UNIT_BYTES * u;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rW, live ? (int)(base + 16 * ((q + rot) & 3)) : (int)OOB, 0, 0);
            wq[slot][q] = make_uint4(v.x, v.y, v.z, v.w);
        }
        // weight scale of the unit's group (g = 256: u/2; one group or mixed: 0)
        const int j = (GM == 1 && !MIXED) ? u : (GM == 2 ? u >> 1 : 0);
        ws[slot] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                 rS, live ? (int)(((uint32_t)n * a.Gw + j) * 4) : (int)OOB, 0, 0));
    };
    // (the activation loads go out first, ahead of the weights: their wait
    // then leaves the weight loads in flight)

    // --- activation rows (rows past M zero) and their scales into LDS ---
    float* lsa = reinterpret_cast<float*>(lds + MR * rowbytes);
    if constexpr (FUSED) {
        // chunk c (8 values) of the MR rows: word c of the packed codes, a
        // group of TPG consecutive chunks (consecutive lanes of one wave); every
        // lane runs every pass, so the groups' lane exchanges see full waves.
        // NB passes' loads are issued before any is used (one L2 round trip
        // per NB passes); chunks of rows past M read as zero (out-of-range
        // buffer offsets).
        using namespace qrule;
        typedef _Float16 half8 __attribute__((ext_vector_type(8)));
        constexpr int TPG = (GM == 2 ? 256 : 128) / 8, NB = 8;
        const int k8 = a.K / 8, n8 = MR * k8, live8 = a.M * k8;
        const __amdgpu_buffer_rsrc_t rX = buffer_of(a.x, (uint32_t)live8 * 16);
        uint32_t* dq = reinterpret_cast<uint32_t*>(lds);
        for (int c0 = 0; c0 < n8; c0 += NB * THREADS) {
            half8 h[NB];
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const int c = c0 + b * THREADS + tid;
                const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rX, c < live8 ? c * 16 : (int)OOB, 0, 0);
                h[b] = __builtin_bit_cast(half8, v);
            }
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const int c = c0 + b * THREADS + tid;
                const float amax = group_max<TPG>(absmax8(h[b]));
                const float scale = amax / 7.0f;
                const bool nz = amax != 0.0f;
                const uint32_t word = quantize8(h[b], scale, nz);
                if (c < n8) {
                    dq[c] = word;
                    if (c % TPG == 0) lsa[c / TPG] = nz ? scale : 0.0f;
                }
            }
        }
    } else {
        // the first NA chunks of this thread in registers, then the first
        // weight loads, then the stores (and any chunks beyond NA)
        constexpr int NA = 4;
        const uint4* src = reinterpret_cast<const uint4*>(a.qa);
        uint4* dst = reinterpret_cast<uint4*>(lds);
        const int nq = MR * (int)rowbytes / 16, live_q = a.lds_qa / 16;
        uint4 av[NA];
        float sv = 0.0f;
#pragma unroll
        for (int c = 0; c < NA; ++c) {
            const int i = tid + c * THREADS;
            av[c] = i < live_q ? src[i] : make_uint4(0, 0, 0, 0);
        }
        if (tid < MR * a.Ga) sv = tid < a.M * a.Ga ? a.sa[tid] : 0.0f;
#pragma unroll
        for (int k = 0; k < PF - 1; ++k) issue(k, k);
#pragma unroll
        for (int c = 0; c < NA; ++c) {
            const int i = tid + c * THREADS;
            if (i < nq) dst[i] = av[c];
        }
        if (tid < MR * a.Ga) lsa[tid] = sv;
        for (int i = tid + NA * THREADS; i < nq; i += THREADS) dst[i] = i < live_q ? src[i] : make_uint4(0, 0, 0, 0);
        for (int i = tid + THREADS; i < MR * a.Ga; i += THREADS) lsa[i] = i < a.M * a.Ga ? a.sa[i] : 0.0f;
    }
    if constexpr (FUSED) {
#pragma unroll
        for (int k = 0; k < PF - 1; ++k) issue(k, k);
    }
    __syncthreads();

    float acc[MR];
    int pint[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        acc[m] = 0.0f;
        pint[m] = 0;
    }

    for (int i0 = 0; i0 < items; i0 += PF)
#pragma unroll
    for (int k = 0; k < PF; ++k) {
        const int i = i0 + k;
        if (i >= items) break;
        issue((k + PF - 1) % PF, i + PF - 1);
        const int r = i / passes, p = i - r * passes;
        const int n = gwave + nwaves * r;
        const int u = lane + 64 * p;
        const bool live = u < a.U;
        const int ja = (a.ga == UNIT) ? u : (GM == 2 ? u >> 1 : 0);   // activation group of the unit
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            // exact int32 sum of the unit's 128 products (16 dot8)
            int P = 0;
            const uint8_t* arow = lds + m * rowbytes + UNIT_BYTES * (live ? u : 0);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint4 av = *reinterpret_cast<const uint4*>(arow + 16 * ((q + rot) & 3));
                const uint4 wv = wq[k][q];
                P = __builtin_amdgcn_sdot8((int)av.x, (int)wv.x, P, false);
                P = __builtin_amdgcn_sdot8((int)av.y, (int)wv.y, P, false);
                P = __builtin_amdgcn_sdot8((int)av.z, (int)wv.z, P, false);
                P = __builtin_amdgcn_sdot8((int)av.w, (int)wv.w, P, false);
            }
            if (GM == 0) {
                pint[m] += P;
            } else {
                if (GM == 2) P += __shfl_xor(P, 1, 64);   // the pair of units of a group
                const bool owner = live && (GM == 1 || (lane & 1) == 0);
                const float sa = owner ? lsa[m * a.Ga + ja] : 0.0f;
                const float S = MIXED ? sa : sa * ws[k];
                acc[m] = fmaf(S, (float)P, acc[m]);
                if (DEBUG_P && owner && m < a.M)
                    if (int32_t* d = psum_at(a.psum, a.prows, m, n, a.N, a.G, GM == 2 ? (u >> 1) : u)) *d = P;
            }
        }
        if (p == passes - 1) {
            // the row is done: lane sums -> Y[m, n]
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                float v;
                if (GM == 0) {
                    const int Pt = wave_sum_int(pint[m]);
                    const float S = lsa[m * a.Ga] * ws[k];
                    v = S * (float)Pt;
                    if (DEBUG_P && lane == 0 && m < a.M)
                        if (int32_t* d = psum_at(a.psum, a.prows, m, n, a.N, 1, 0)) *d = Pt;
                    pint[m] = 0;
                } else {
                    v = wave_sum(acc[m]);
                    if (MIXED) v *= ws[k];
                    acc[m] = 0.0f;
                }
                // keep the fp32 value: y16 is the fp16 rounding of y32
                asm volatile("" : "+v"(v));
                if (lane == 0 && m < a.M) {
                    const int64_t o = (int64_t)m * a.N + n;
                    a.y16[o] = (_Float16)v;
                    if (a.y32) a.y32[o] = v;
                }
            }
        }
    }
}

template <int MR>
hipError_t launch_mr(const GemvArgs& g, int gm, bool mixed, bool dbg, hipStream_t stream, bool fused = false)
{
    const int blocks = (g.N + WAVES - 1) / WAVES < 256 ? (g.N + WAVES - 1) / WAVES : 256;
    const size_t lds = (size_t)MR * g.K / 2 + (size_t)MR * g.Ga * 4;
    // dynamic LDS above 64 KB has to be allowed per kernel
#define APEX4_GEMV_K(GM_, MX, DB, FU)                                                            \
    do {                                                                                        \
        if (lds > 65536) {                                                                      \
            const hipError_t e = hipFuncSetAttribute(                                           \
                reinterpret_cast<const void*>(&gemm_gemv_kernel<MR, GM_, MX, DB, FU>),          \
                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);                          \
            if (e != hipSuccess) return e;                                                      \
        }                                                                                       \
        gemm_gemv_kernel<MR, GM_, MX, DB, FU><<<blocks, THREADS, lds, stream>>>(g);             \
    } while (0)
#define APEX4_GEMV(GM_, MX, DB) APEX4_GEMV_K(GM_, MX, DB, false)
    if (fused) {
        // (groups of 128 or 256, mixed with 128; no debug sums)
        if (mixed) APEX4_GEMV_K(1, true, false, true);
        else if (gm == 2) APEX4_GEMV_K(2, false, false, true);
        else APEX4_GEMV_K(1, false, false, true);
    } else if (mixed) {
        if (dbg) APEX4_GEMV(1, true, true);
        else APEX4_GEMV(1, true, false);
    } else if (gm == 1) {
        if (dbg) APEX4_GEMV(1, false, true);
        else APEX4_GEMV(1, false, false);
    } else if (gm == 2) {
        if (dbg) APEX4_GEMV(2, false, true);
        else APEX4_GEMV(2, false, false);
    } else {
        if (dbg) APEX4_GEMV(0, false, true);
        else APEX4_GEMV(0, false, false);
    }
#undef APEX4_GEMV
#undef APEX4_GEMV_K
    return hipGetLastError();
}

int rows_template(int M) { return M <= 1 ? 1 : M <= 2 ? 2 : 4; }

}  // namespace

bool gemv_supports(const GemmProblem& p)
{
    if (p.M < 1 || p.M > 4) return false;
    const int gs = p.ga < p.gw ? p.ga : p.gw;
    const bool mixed = p.gw == p.K && p.ga != p.gw;
    // groups of 128, 256, one group over K; mixed mode with activation groups of 128
    if (mixed) {
        if (p.ga != UNIT) return false;
    } else if (p.ga != p.gw || !(gs == UNIT || gs == 2 * UNIT || gs == p.K) || p.K % UNIT != 0) {
        return false;
    }
    // 32-bit buffer offsets; activation rows and scales must fit in LDS
    const uint64_t wbytes = (uint64_t)p.N * (p.K / 2), sbytes = (uint64_t)p.N * (p.K / p.gw) * 4;
    const int mr = rows_template(p.M);
    const uint64_t lds = (uint64_t)mr * p.K / 2 + (uint64_t)mr * (p.K / p.ga) * 4;
    return wbytes < OOB && sbytes < OOB && lds <= 160 * 1024;
}

bool gemv_fused_supports(const GemmProblem& p)
{
    // the row-streaming kernel with 1 or 2 rows, activation groups of 128 or
    // 256 (one group over K would need a row-wide maximum first), K up to
    // 8192: every workgroup reads the fp16 rows (4x the bytes of their codes)
    // before its weight stream starts, and at the per-CU fetch rate of the
    // stream that costs more than the separate quantization launch beyond
    // that (70B down-projection, K = 28672: 27.3 us fused, 25.8 us as two
    // launches; up-projection, K = 8192: 24.8 us and 24.9 us)
    return p.M >= 1 && p.M <= 2 && p.K <= 8192 && gemv_supports(p) && (p.ga == UNIT || p.ga == 2 * UNIT);
}

hipError_t launch_gemm_gemv_fused(const GemmProblem& p, const void* x_f16, hipStream_t stream)
{
    GemvArgs g{};
    g.qa = nullptr;
    g.sa = nullptr;
    g.x = static_cast<const _Float16*>(x_f16);
    g.qw = p.qw;
    g.sw = p.sw;
    g.M = p.M;
    g.N = p.N;
    g.K = p.K;
    g.Ga = p.K / p.ga;
    g.Gw = p.K / p.gw;
    g.ga = p.ga;
    const int gs = p.ga < p.gw ? p.ga : p.gw;
    g.G = p.K / gs;
    g.U = p.K / UNIT;
    g.lds_qa = p.M * (p.K / 2);
    g.y16 = static_cast<_Float16*>(p.y16);
    g.y32 = p.y32;
    g.psum = nullptr;
    const bool mixed = p.gw == p.K && p.ga != p.gw;
    const int gm = gs == 2 * UNIT ? 2 : 1;
    if (p.M == 1) return launch_mr<1>(g, gm, mixed, false, stream, true);
    return launch_mr<2>(g, gm, mixed, false, stream, true);
}

hipError_t launch_gemm_gemv(const GemmProblem& p, hipStream_t stream)
{
    GemvArgs g{};
    g.qa = p.qa;
    g.sa = p.sa;
    g.qw = p.qw;
    g.sw = p.sw;
    g.M = p.M;
    g.N = p.N;
    g.K = p.K;
    g.Ga = p.K / p.ga;
    g.Gw = p.K / p.gw;
    g.ga = p.ga;
    const int gs = p.ga < p.gw ? p.ga : p.gw;
    g.G = p.K / gs;
    g.U = p.K / UNIT;
    g.lds_qa = p.M * (p.K / 2);
    g.y16 = static_cast<_Float16*>(p.y16);
    g.y32 = p.y32;
    g.psum = p.psum;
    g.prows = p.prows;
    const bool mixed = p.gw == p.K && p.ga != p.gw;
    const int gm = gs == p.K && !mixed ? 0 : gs == 2 * UNIT ? 2 : 1;
    const bool dbg = p.psum != nullptr;
    switch (rows_template(p.M)) {
    case 1: return launch_mr<1>(g, gm, mixed, dbg, stream);
    case 2: return launch_mr<2>(g, gm, mixed, dbg, stream);
    default: return launch_mr<4>(g, gm, mixed, dbg, stream);
    }
}

}  // namespace apex4
