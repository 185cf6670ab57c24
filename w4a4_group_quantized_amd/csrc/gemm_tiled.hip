// W4A4 GEMM with per-group dequantization on gfx950 (CDNA4): the tiled kernel
// for row counts where the product is compute-bound (prefill-shaped calls).
//
// The computation is the APEX4 page's (Abstract): INT4 x INT4 products summed
// exactly per K-group on the matrix units, then every group's integer sum is
// rescaled by s_a*s_w and accumulated in fp32 on the vector ALUs.  gfx950 has
// no INT4 matrix instruction, so each nibble is widened to an int8 and fed to
// v_mfma_i32_32x32x32_i8.
//
// Nibble widening.  A packed word holds 8 codes c0..c7 (c_i in bits 4i..4i+3).
// (w << 4) & 0xF0F0F0F0 puts c0,c2,c4,c6 in the high half of four bytes and
// w & 0xF0F0F0F0 does the same for c1,c3,c5,c7: each byte is then the signed
// int8 16*c, with no sign extension step (3 VALU ops per 8 codes).  Both
// operands are widened the same way, so the MFMA returns 256*P exactly
// (|256*P| <= 256*64*K < 2^31 for K < 2^17) and the factor 2^-8 is folded into
// the activation scale, which is exact.  The even/odd split permutes K inside
// each 16-value half of a 32-value step identically for both operands, so
// every step still sums exactly the products of one group.
//
// Work split.  A workgroup of 4 waves computes a 128x128 tile of Y; each wave a
// 64x64 sub-tile as 2x2 MFMA tiles of 32x32.  K advances in stages of 128
// values.  The widening is done once per workgroup, in the copy from global
// memory to LDS: the vector ALUs are the bottleneck of this method, and doing
// it there instead of after every wave's LDS read halves that work.  A stage
// of A and B is thus held in LDS as int8 (128 bytes per row, rows 144 bytes
// apart so that the 16-byte fragment reads of 16 consecutive rows hit every
// bank once), double-buffered with one barrier per stage; the packed bytes of
// the next stage are fetched into registers (16-byte global loads) while the
// current one is multiplied.
//
// Rescale cadence follows the group size gs = min(g_a, g_w): after every
// K-step (gs = 32), every second step (64), or every gs/128 stages (>= 128).
// In mixed mode (g_w = K) the weight scale is applied once in the epilogue.
#include "internal.h"

namespace apex4 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int KSTAGE = 128;          // K values per stage
constexpr int ROWB = KSTAGE / 2;     // packed bytes per row per stage
constexpr int LDS_STRIDE = 144;      // LDS bytes per row: 128 int8 + 16 padding
constexpr int MAX_SUB = KSTAGE / 32; // scale groups per stage at gs = 32

struct TileArgs {
    const uint8_t* qa;
    const float* sa;
    const uint8_t* qw;
    const float* sw;
    int M, N, K;
    int Ga, Gw;       // scale columns per row: K/ga, K/gw
    int ga, gw, gs;   // group sizes; gs = min(ga, gw)
    int G;            // K / gs
    _Float16* y16;
    float* y32;
    int32_t* psum;
};

__device__ inline uint4 widen_lo(uint4 w)
{
    // the first 16 codes of a 32-code chunk (words w.x, w.y) as 16 int8 (x16)
    return make_uint4((w.x << 4) & 0xF0F0F0F0u, w.x & 0xF0F0F0F0u,
                      (w.y << 4) & 0xF0F0F0F0u, w.y & 0xF0F0F0F0u);
}

__device__ inline uint4 widen_hi(uint4 w)
{
    return make_uint4((w.z << 4) & 0xF0F0F0F0u, w.z & 0xF0F0F0F0u,
                      (w.w << 4) & 0xF0F0F0F0u, w.w & 0xF0F0F0F0u);
}

// Row-in-tile of accumulator register r for this lane (32x32 MFMA output).
__device__ inline int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// GS_STEPS: K-steps (of 32) per group when the group is smaller than a stage
// (1 or 2), or 0 when a group spans whole stages.
template <int GS_STEPS, bool MIXED, bool DEBUG_P>
__global__ __launch_bounds__(256, 2) void gemm_tiled_kernel(TileArgs a)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][BM * LDS_STRIDE];
    __shared__ __attribute__((aligned(16))) uint8_t lds_b[2][BN * LDS_STRIDE];
    constexpr int SUBS = GS_STEPS ? MAX_SUB / GS_STEPS : 1;   // scale groups per stage
    __shared__ __attribute__((aligned(16))) float lds_sa[2][SUBS][BM];
    __shared__ __attribute__((aligned(16))) float lds_sw[2][MIXED ? 1 : SUBS][BN];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
    const int64_t rowbytes = a.K / 2;
    const int stages = a.K / KSTAGE;
    const int nsub = SUBS;
    const int stages_per_group = GS_STEPS ? 1 : a.gs / KSTAGE;

    // --- global -> register staging: 2 chunks (16 packed bytes = one K-step
    // of one row) of A and 2 of B per thread, plus 2 scales of each ---
    uint4 ra[2], rb[2];
    float rsa[2], rsw[2];

    auto load_stage = [&](int t) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int c = tid + 256 * i;
            const int row = c >> 2, s = c & 3;
            const int64_t koff = (int64_t)t * ROWB + s * 16;
            const int am = m0 + row, bn = n0 + row;
            ra[i] = am < a.M ? *reinterpret_cast<const uint4*>(a.qa + am * rowbytes + koff)
                             : make_uint4(0, 0, 0, 0);
            rb[i] = bn < a.N ? *reinterpret_cast<const uint4*>(a.qw + bn * rowbytes + koff)
                             : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int idx = tid + 256 * i;
            const int row = idx & 127, sub = idx >> 7;
            rsa[i] = 0.0f;
            rsw[i] = 0.0f;
            if (sub < nsub) {
                const int k0 = t * KSTAGE + sub * a.gs;
                const int am = m0 + row, bn = n0 + row;
                if (am < a.M) rsa[i] = a.sa[(int64_t)am * a.Ga + k0 / a.ga] * 0.00390625f;
                if (!MIXED && bn < a.N) rsw[i] = a.sw[(int64_t)bn * a.Gw + k0 / a.gw];
            }
        }
    };

    // widen the staged chunks and store them: K-step s of a row occupies bytes
    // [32s, 32s+32) of the row, first half (codes 0..15) then second half
    auto store_stage = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int c = tid + 256 * i;
            const int row = c >> 2, s = c & 3;
            const int o = row * LDS_STRIDE + 32 * s;
            *reinterpret_cast<uint4*>(&lds_a[buf][o]) = widen_lo(ra[i]);
            *reinterpret_cast<uint4*>(&lds_a[buf][o + 16]) = widen_hi(ra[i]);
            *reinterpret_cast<uint4*>(&lds_b[buf][o]) = widen_lo(rb[i]);
            *reinterpret_cast<uint4*>(&lds_b[buf][o + 16]) = widen_hi(rb[i]);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int idx = tid + 256 * i;
            const int row = idx & 127, sub = idx >> 7;
            if (sub < nsub) {
                lds_sa[buf][sub][row] = rsa[i];
                if (!MIXED) lds_sw[buf][sub][row] = rsw[i];
            }
        }
    };

    float acc[2][2][16];
    v16i P[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mt][nt][r] = 0.0f;
        }

    // Rescale the finished group held in P (scale-group `sub` of stage buffer
    // `buf`, global group index j) into acc.
    auto rescale = [&](int buf, int sub, int j) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            float sa[16];
            const float* sp = &lds_sa[buf][sub][wm * 64 + mt * 32 + 4 * (lane >> 5)];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 v = *reinterpret_cast<const float4*>(sp + 8 * q);
                sa[4 * q + 0] = v.x;
                sa[4 * q + 1] = v.y;
                sa[4 * q + 2] = v.z;
                sa[4 * q + 3] = v.w;
            }
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                float sw = 1.0f;
                if (!MIXED) sw = lds_sw[buf][sub][wn * 64 + nt * 32 + (lane & 31)];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float S = MIXED ? sa[r] : sa[r] * sw;
                    acc[mt][nt][r] = fmaf(S, (float)P[mt][nt][r], acc[mt][nt][r]);
                }
                if (DEBUG_P) {
                    const int n = n0 + wn * 64 + nt * 32 + (lane & 31);
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int m = m0 + wm * 64 + mt * 32 + acc_row(r, lane);
                        if (m < a.M && n < a.N)
                            a.psum[((int64_t)m * a.N + n) * a.G + j] = P[mt][nt][r] >> 8;
                    }
                }
            }
        }
    };

    load_stage(0);
    store_stage(0);
    __syncthreads();

    for (int t = 0; t < stages; ++t) {
        const int buf = t & 1;
        if (t + 1 < stages) load_stage(t + 1);

        const uint8_t* la = lds_a[buf] + (wm * 64 + (lane & 31)) * LDS_STRIDE + 16 * (lane >> 5);
        const uint8_t* lb = lds_b[buf] + (wn * 64 + (lane & 31)) * LDS_STRIDE + 16 * (lane >> 5);
        // small groups rescale inside this loop; keeping it rolled there keeps
        // the fragments of only one step live across a rescale
#pragma unroll (GS_STEPS ? 1 : 4)
        for (int s = 0; s < 4; ++s) {
            v4i fa[2], fb[2];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
                fa[mt] = *reinterpret_cast<const v4i*>(la + mt * 32 * LDS_STRIDE + 32 * s);
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
                fb[nt] = *reinterpret_cast<const v4i*>(lb + nt * 32 * LDS_STRIDE + 32 * s);
            // the first K-step of a group starts from a zero accumulator (an
            // inline constant), so no registers are spent clearing P
            const bool first = GS_STEPS ? (s % GS_STEPS == 0) : (s == 0 && t % stages_per_group == 0);
            if (first) {
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt)
                        P[mt][nt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[mt], fb[nt], v16i{},
                                                                         0, 0, 0);
            } else {
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt)
                        P[mt][nt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[mt], fb[nt], P[mt][nt],
                                                                         0, 0, 0);
            }
            if (GS_STEPS == 1) rescale(buf, s, t * MAX_SUB + s);
            if (GS_STEPS == 2 && (s & 1)) rescale(buf, s >> 1, t * (MAX_SUB / 2) + (s >> 1));
        }
        if (GS_STEPS == 0 && (t + 1) % stages_per_group == 0) rescale(buf, 0, t / stages_per_group);

        if (t + 1 < stages) store_stage(buf ^ 1);
        __syncthreads();
    }

    // --- epilogue: (mixed: x s_w[n]) -> fp16 (RNE) and optional fp32 ---
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const int n = n0 + wn * 64 + nt * 32 + (lane & 31);
            float swn = 1.0f;
            if (MIXED && n < a.N) swn = a.sw[n];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm * 64 + mt * 32 + acc_row(r, lane);
                if (m < a.M && n < a.N) {
                    float v = MIXED ? acc[mt][nt][r] * swn : acc[mt][nt][r];
                    // keep the fp32 value as is: without this the multiply and the
                    // fp16 conversion may fuse into one rounding, and y16 would no
                    // longer be the fp16 rounding of y32
                    asm volatile("" : "+v"(v));
                    const int64_t o = (int64_t)m * a.N + n;
                    a.y16[o] = (_Float16)v;
                    if (a.y32) a.y32[o] = v;
                }
            }
        }
}

template <int GS_STEPS>
void launch_tiled_mode(const TileArgs& t, bool mixed, hipStream_t stream)
{
    dim3 grid((t.N + BN - 1) / BN, (t.M + BM - 1) / BM);
    const bool dbg = t.psum != nullptr;
    if (mixed) {
        if (dbg) gemm_tiled_kernel<GS_STEPS, true, true><<<grid, 256, 0, stream>>>(t);
        else gemm_tiled_kernel<GS_STEPS, true, false><<<grid, 256, 0, stream>>>(t);
    } else {
        if (dbg) gemm_tiled_kernel<GS_STEPS, false, true><<<grid, 256, 0, stream>>>(t);
        else gemm_tiled_kernel<GS_STEPS, false, false><<<grid, 256, 0, stream>>>(t);
    }
}

}  // namespace

hipError_t launch_gemm_tiled(const GemmProblem& p, hipStream_t stream)
{
    TileArgs t;
    t.qa = p.qa;
    t.sa = p.sa;
    t.qw = p.qw;
    t.sw = p.sw;
    t.M = p.M;
    t.N = p.N;
    t.K = p.K;
    t.ga = p.ga;
    t.gw = p.gw;
    t.gs = p.ga < p.gw ? p.ga : p.gw;
    t.Ga = p.K / p.ga;
    t.Gw = p.K / p.gw;
    t.G = p.K / t.gs;
    t.y16 = static_cast<_Float16*>(p.y16);
    t.y32 = p.y32;
    t.psum = p.psum;
    const bool mixed = (p.gw == p.K) && (p.ga != p.gw);
    if (t.gs == 32)
        launch_tiled_mode<1>(t, mixed, stream);
    else if (t.gs == 64)
        launch_tiled_mode<2>(t, mixed, stream);
    else
        launch_tiled_mode<0>(t, mixed, stream);
    return hipGetLastError();
}

}  // namespace apex4
