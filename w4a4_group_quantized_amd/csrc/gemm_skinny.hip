// W4A4 GEMM for few rows (decode-shaped calls, M <= 64) on gfx950.
//
// With a handful of tokens the product is bound by reading the packed weights
// from HBM once (the blog page "Why INT4 Weight-Only Quantization Doesn't Speed
// Up Prefill" works through this: intensity 2B/b FLOP per byte at B tokens),
// so this kernel is organised around streaming qw, not around the matrix
// units.  The arithmetic is the same as the tiled kernel's: nibbles widened to
// int8 (x16), exact int32 group sums from v_mfma_i32_16x16x64_i8, fp32
// rescale by s_a*s_w on the vector ALUs.
//
// Work split.  A workgroup of 8 waves owns 32 output columns and all M rows
// (16x16 MFMA tiles: ceil(M/16) row tiles, 2 column tiles).  The waves split
// the K-groups among themselves (wave w takes groups w, w+8, ...), so every
// wave streams 32 weight rows x 64 bytes per 128-value chunk with 16-byte
// loads while the other waves read the neighbouring chunks of the same rows.
// Each wave keeps the loads of the next PREFETCH chunks in flight.  At the end
// the eight partial fp32 tiles are summed through LDS in a fixed order.  When
// the whole row is one group (per-channel scales on both operands) the waves
// instead split its chunks and sum the int32 partial sums exactly before the
// single rescale.
//
// K order inside a chunk: lane block kb (lanes 16kb..16kb+15) holds the 32
// codes of bytes [16kb, 16kb+16); the first 16 feed K-step 0 and the last 16
// K-step 1.  The same assignment is used for both operands, so each MFMA sums
// the products of one chunk, i.e. of one group (groups are >= 128 here).
#include "internal.h"

namespace apex4 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int WAVES = 8;
constexpr int BN = 32;          // output columns per workgroup
constexpr int CHUNK = 128;      // K values per chunk (64 packed bytes per row)
constexpr int PREFETCH = 4;     // chunks in flight per wave

struct SkinnyArgs {
    const uint8_t* qa;
    const float* sa;
    const uint8_t* qw;
    const float* sw;
    int M, N, K;
    int Ga, Gw;       // scale columns per row
    int ga, gw, gs;   // group sizes, gs = min(ga, gw) >= 128
    int G;            // K / gs
    _Float16* y16;
    float* y32;
    int32_t* psum;
};

__device__ inline v4i widen_lo(uint4 w)
{
    v4i r;
    r[0] = (int)((w.x << 4) & 0xF0F0F0F0u);
    r[1] = (int)(w.x & 0xF0F0F0F0u);
    r[2] = (int)((w.y << 4) & 0xF0F0F0F0u);
    r[3] = (int)(w.y & 0xF0F0F0F0u);
    return r;
}

__device__ inline v4i widen_hi(uint4 w)
{
    v4i r;
    r[0] = (int)((w.z << 4) & 0xF0F0F0F0u);
    r[1] = (int)(w.z & 0xF0F0F0F0u);
    r[2] = (int)((w.w << 4) & 0xF0F0F0F0u);
    r[3] = (int)(w.w & 0xF0F0F0F0u);
    return r;
}

// MT: 16-row tiles (ceil(M/16)).  ONE_GROUP: gs == K, waves split the chunks
// of the single group and add their int32 sums before rescaling.
template <int MT, bool MIXED, bool DEBUG_P, bool ONE_GROUP>
__global__ __launch_bounds__(512) void gemm_skinny_kernel(SkinnyArgs a)
{
    // cross-wave reduction buffer: [wave][mt][nt][r][lane]
    __shared__ float red[WAVES][MT][2][4][64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int li = lane & 15, kb = lane >> 4;
    const int n0 = blockIdx.x * BN;
    const int64_t rowbytes = a.K / 2;
    const int chunks_per_group = a.gs / CHUNK;
    const int total_chunks = a.K / CHUNK;

    // row / column this lane loads
    const uint8_t* pa[MT];
    bool va[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int m = 16 * mt + li;
        va[mt] = m < a.M;
        pa[mt] = a.qa + (int64_t)(va[mt] ? m : 0) * rowbytes + 16 * kb;
    }
    const uint8_t* pb[2];
    bool vb[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const int n = n0 + 16 * nt + li;
        vb[nt] = n < a.N;
        pb[nt] = a.qw + (int64_t)(vb[nt] ? n : 0) * rowbytes + 16 * kb;
    }

    // this wave's chunk sequence: i -> chunk index
    //   grouped:   groups j = wave, wave+8, ..., each contributing its chunks
    //   one group: chunks wave, wave+8, ...
    const int my_groups = ONE_GROUP ? 0 : (a.G > wave ? (a.G - wave + WAVES - 1) / WAVES : 0);
    const int n_chunks = ONE_GROUP ? (total_chunks > wave ? (total_chunks - wave + WAVES - 1) / WAVES : 0)
                                   : my_groups * chunks_per_group;
    auto chunk_of = [&](int i) -> int {
        if (ONE_GROUP) return wave + WAVES * i;
        const int jj = i / chunks_per_group;
        return (wave + WAVES * jj) * chunks_per_group + (i - jj * chunks_per_group);
    };

    uint4 bufA[PREFETCH][MT], bufB[PREFETCH][2];
    auto issue = [&](int slot_i, int i) {
        // slot_i is a compile-time slot index after unrolling
        if (i < n_chunks) {
            const int64_t off = (int64_t)chunk_of(i) * (CHUNK / 2);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                bufA[slot_i][mt] = va[mt] ? *reinterpret_cast<const uint4*>(pa[mt] + off)
                                          : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
                bufB[slot_i][nt] = vb[nt] ? *reinterpret_cast<const uint4*>(pb[nt] + off)
                                          : make_uint4(0, 0, 0, 0);
        }
    };

    float acc[MT][2][4];
    v4i P[MT][2];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[mt][nt][r] = 0.0f;
            P[mt][nt] = v4i{};
        }

#pragma unroll
    for (int k = 0; k < PREFETCH - 1; ++k) issue(k, k);

    for (int i0 = 0; i0 < n_chunks; i0 += PREFETCH) {
#pragma unroll
        for (int k = 0; k < PREFETCH; ++k) {
            const int i = i0 + k;
            issue((k + PREFETCH - 1) % PREFETCH, i + PREFETCH - 1);
            if (i < n_chunks) {
                const int u = ONE_GROUP ? 1 : i % chunks_per_group;   // chunk within group
                const bool first = ONE_GROUP ? (i == 0) : (u == 0);
                v4i fa[MT][2], fb[2][2];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    fa[mt][0] = widen_lo(bufA[k][mt]);
                    fa[mt][1] = widen_hi(bufA[k][mt]);
                }
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    fb[nt][0] = widen_lo(bufB[k][nt]);
                    fb[nt][1] = widen_hi(bufB[k][nt]);
                }
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) {
                        v4i c = first ? v4i{} : P[mt][nt];
                        c = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[mt][0], fb[nt][0], c, 0, 0, 0);
                        P[mt][nt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[mt][1], fb[nt][1], c, 0, 0, 0);
                    }
                if (!ONE_GROUP && u == chunks_per_group - 1) {
                    // the group is complete: rescale into acc
                    const int j = wave + WAVES * (i / chunks_per_group);
                    const int kg = j * a.gs;
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        float sa[4];
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int m = 16 * mt + 4 * kb + r;
                            sa[r] = m < a.M ? a.sa[(int64_t)m * a.Ga + kg / a.ga] * 0.00390625f : 0.0f;
                        }
#pragma unroll
                        for (int nt = 0; nt < 2; ++nt) {
                            const int n = n0 + 16 * nt + li;
                            float sw = 1.0f;
                            if (!MIXED) sw = vb[nt] ? a.sw[(int64_t)n * a.Gw + kg / a.gw] : 0.0f;
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                const float S = MIXED ? sa[r] : sa[r] * sw;
                                acc[mt][nt][r] = fmaf(S, (float)P[mt][nt][r], acc[mt][nt][r]);
                            }
                            if (DEBUG_P && vb[nt]) {
#pragma unroll
                                for (int r = 0; r < 4; ++r) {
                                    const int m = 16 * mt + 4 * kb + r;
                                    if (m < a.M)
                                        a.psum[((int64_t)m * a.N + n) * a.G + j] = P[mt][nt][r] >> 8;
                                }
                            }
                        }
                    }
                }
            }
        }
    }

    if (ONE_GROUP) {
        // exact int32 sum of the waves' partial sums, then one rescale
        int* redi = reinterpret_cast<int*>(&red[0][0][0][0][0]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    redi[(((wave * MT + mt) * 2 + nt) * 4 + r) * 64 + lane] = n_chunks ? P[mt][nt][r] : 0;
        __syncthreads();
        if (wave == 0) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    const int n = n0 + 16 * nt + li;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        int p = 0;
                        for (int w = 0; w < WAVES; ++w)
                            p += redi[(((w * MT + mt) * 2 + nt) * 4 + r) * 64 + lane];
                        const int m = 16 * mt + 4 * kb + r;
                        if (m < a.M && n < a.N) {
                            const float S = a.sa[m] * 0.00390625f * a.sw[n];
                            float v = S * (float)p;
                            asm volatile("" : "+v"(v));
                            const int64_t o = (int64_t)m * a.N + n;
                            a.y16[o] = (_Float16)v;
                            if (a.y32) a.y32[o] = v;
                            if (DEBUG_P) a.psum[o] = p >> 8;
                        }
                    }
                }
        }
        return;
    }

    // sum the eight partial tiles in a fixed order, then write
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[wave][mt][nt][r][lane] = acc[mt][nt][r];
    __syncthreads();
    for (int o = tid; o < MT * 2 * 4 * 64; o += WAVES * 64) {
        const int ln = o & 63, r = (o >> 6) & 3, nt = (o >> 8) & 1, mt = o >> 9;
        const int m = 16 * mt + 4 * (ln >> 4) + r;
        const int n = n0 + 16 * nt + (ln & 15);
        if (m < a.M && n < a.N) {
            float v = 0.0f;
#pragma unroll
            for (int w = 0; w < WAVES; ++w) v += red[w][mt][nt][r][ln];
            if (MIXED) v *= a.sw[n];
            asm volatile("" : "+v"(v));
            const int64_t off = (int64_t)m * a.N + n;
            a.y16[off] = (_Float16)v;
            if (a.y32) a.y32[off] = v;
        }
    }
}

template <int MT>
void launch_mt(const SkinnyArgs& s, bool mixed, bool dbg, bool one, hipStream_t stream)
{
    dim3 grid((s.N + BN - 1) / BN);
#define APEX4_SKINNY(MX, DB, ONE) gemm_skinny_kernel<MT, MX, DB, ONE><<<grid, WAVES * 64, 0, stream>>>(s)
    if (one) {
        if (dbg) APEX4_SKINNY(false, true, true);
        else APEX4_SKINNY(false, false, true);
    } else if (mixed) {
        if (dbg) APEX4_SKINNY(true, true, false);
        else APEX4_SKINNY(true, false, false);
    } else {
        if (dbg) APEX4_SKINNY(false, true, false);
        else APEX4_SKINNY(false, false, false);
    }
#undef APEX4_SKINNY
}

}  // namespace

bool skinny_supports(const GemmProblem& p)
{
    const int gs = p.ga < p.gw ? p.ga : p.gw;
    return p.M >= 1 && p.M <= 64 && gs >= CHUNK;
}

hipError_t launch_gemm_skinny(const GemmProblem& p, hipStream_t stream)
{
    SkinnyArgs s;
    s.qa = p.qa;
    s.sa = p.sa;
    s.qw = p.qw;
    s.sw = p.sw;
    s.M = p.M;
    s.N = p.N;
    s.K = p.K;
    s.ga = p.ga;
    s.gw = p.gw;
    s.gs = p.ga < p.gw ? p.ga : p.gw;
    s.Ga = p.K / p.ga;
    s.Gw = p.K / p.gw;
    s.G = p.K / s.gs;
    s.y16 = static_cast<_Float16*>(p.y16);
    s.y32 = p.y32;
    s.psum = p.psum;
    const bool mixed = (p.gw == p.K) && (p.ga != p.gw);
    const bool one = s.gs == p.K;
    const bool dbg = p.psum != nullptr;
    const int mt = (p.M + 15) / 16;
    switch (mt) {
    case 1: launch_mt<1>(s, mixed, dbg, one, stream); break;
    case 2: launch_mt<2>(s, mixed, dbg, one, stream); break;
    case 3: launch_mt<3>(s, mixed, dbg, one, stream); break;
    default: launch_mt<4>(s, mixed, dbg, one, stream); break;
    }
    return hipGetLastError();
}

}  // namespace apex4
