// W4A4 GEMM with per-group dequantization on gfx950 (CDNA4): the tiled kernel
// for row counts where the product is compute-bound (prefill-shaped calls).
//
// The computation is the APEX4 page's (Abstract): INT4 x INT4 products summed
// exactly per K-group on the matrix units, then every group's integer sum is
// rescaled by s_a*s_w and accumulated in fp32 on the vector ALUs.  That
// rescale is the method's bottleneck on this chip as on the page's A100: the
// int8 MFMA finishes a 32x32x128 group in 128 cycles, while the vector ALU
// needs 4 cycles per instruction for the 16 outputs a lane holds per tile.
// Everything below is arranged to spend as few vector instructions per MFMA
// as possible.
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
// Work split.  A workgroup of 8 waves computes a 256x128 tile of Y; each wave a
// 64x64 sub-tile as 2x2 MFMA tiles of 32x32 (v_mfma_i32_32x32x32_i8).  K
// advances in stages of 128 values.  The widening is done once per workgroup,
// in the copy from global memory to LDS, so a stage of A and B is held in LDS
// as int8 (128 bytes per row, rows 144 bytes apart so that the 16-byte
// fragment reads of 16 consecutive rows hit every bank once), double-buffered
// with one barrier per stage; the packed bytes of the stage after next are
// fetched into registers (16-byte global loads) while the current one is
// multiplied.
//
// Group rescale, equal group sizes.  The products S = s_a[m]*s_w[n] of
// a 32x32 tile come from one v_mfma_f32_32x32x16_bf16 instead of 16 vector
// multiplies per lane: each scale is split exactly into three bf16 pieces
// s = x0 + x1 + x2 (8 significant bits each, truncation), and the six largest
// cross products x_p*y_q (p+q <= 2) fill six of the 16 K slots; the three
// dropped ones are below 2^-23 of S.  The pieces are formed once per
// workgroup by the threads that stage the scales, and stored in LDS in the
// operand layout, one table per group of the stage (4 at g = 32, 2 at
// g = 64).  The vector work left per output and group is one int->fp32
// conversion and one fma.  Mixed mode (per-channel weights) needs no product:
// it rescales with s_a from a plain fp32 table and applies s_w once in the
// epilogue.
//
// Rescale cadence follows the group size gs = min(g_a, g_w): after every
// K-step (gs = 32), every second step (64), or every gs/128 stages (>= 128).
#include "internal.h"

namespace apex4 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

#ifndef APEX4_TILED_BM
#define APEX4_TILED_BM 256
#endif
constexpr int BM = APEX4_TILED_BM;   // 256: 8 waves, one workgroup per CU; 128: 4 waves, two
constexpr int BN = 128;
constexpr int THREADS = BM * 2;     // waves as a (BM/64) x 2 grid of 64x64 sub-tiles
constexpr int BCH = BN * 4 / THREADS;   // B chunks (16 packed bytes) per thread per stage
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
    PsumRows prows;
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

// bf16 bits of the truncation of x (x's top 16 bits)
__device__ inline uint32_t bf16_trunc_bits(float x) { return __builtin_bit_cast(uint32_t, x) >> 16; }

// Exact split s = x0 + x1 + x2 into three bf16 values (truncation at each step).
__device__ inline void split3(float s, uint32_t& x0, uint32_t& x1, uint32_t& x2)
{
    x0 = bf16_trunc_bits(s);
    const float r1 = s - __builtin_bit_cast(float, x0 << 16);
    x1 = bf16_trunc_bits(r1);
    const float r2 = r1 - __builtin_bit_cast(float, x1 << 16);
    x2 = bf16_trunc_bits(r2);
}

// Row-in-tile of accumulator register r for this lane (32x32 MFMA output).
__device__ inline int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// GS_STEPS: K-steps (of 32) per group: 1 or 2 (groups of 32 or 64), 4 (one
// group per stage, g = 128), or 0 when a group spans several stages.  SPLIT:
// the scale product comes from the bf16 MFMA (equal group sizes).
template <int GS_STEPS, bool MIXED, bool DEBUG_P>
__global__ __launch_bounds__(THREADS, 2) void gemm_tiled_kernel(TileArgs a)
{
    constexpr bool SPLIT = !MIXED;
    constexpr bool SMALL = GS_STEPS == 1 || GS_STEPS == 2;    // several groups per stage
    constexpr int SUBS = SMALL ? MAX_SUB / GS_STEPS : 1;       // scale groups per stage
    constexpr int NS = (BM * SUBS + THREADS - 1) / THREADS;    // scale values per thread per operand
    __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][BM * LDS_STRIDE];
    __shared__ __attribute__((aligned(16))) uint8_t lds_b[2][BN * LDS_STRIDE];
    // Scale tables, per stage buffer: fp32 scales [SUBS][BM] and [SUBS][BN]
    // (small groups, mixed mode), or for SPLIT the bf16 split operands, one
    // 16-byte row per tile row (the last dword always 0).
    constexpr int TAB_A = SUBS * BM * (SPLIT ? 4 : 1);                // floats / dwords per buffer
    constexpr int TAB_B = MIXED ? 0 : SUBS * BN * (SPLIT ? 4 : 1);
    __shared__ __attribute__((aligned(16))) float lds_tab[2 * (TAB_A + TAB_B)];
    auto sa_tab = [&](int buf, int sub) -> float* { return lds_tab + buf * TAB_A + sub * BM; };
    auto sw_tab = [&](int buf, int sub) -> float* { return lds_tab + 2 * TAB_A + buf * TAB_B + sub * BN; };
    auto spa_tab = [&](int buf, int sub) -> uint4* {
        return reinterpret_cast<uint4*>(lds_tab + buf * TAB_A + sub * BM * 4);
    };
    auto spb_tab = [&](int buf, int sub) -> uint4* {
        return reinterpret_cast<uint4*>(lds_tab + 2 * TAB_A + buf * TAB_B + sub * BN * 4);
    };
    // A zero row for lanes 32..63 of the split-operand MFMA (their K slots
    // 8..15 are unused): the padding of row 0 of A buffer 0, which no stage
    // ever writes.
    uint4* const lds_zero = reinterpret_cast<uint4*>(&lds_a[0][128]);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
    const int64_t rowbytes = a.K / 2;
    const int stages = a.K / KSTAGE;
    const int stages_per_group = GS_STEPS ? 1 : a.gs / KSTAGE;   // (GS_STEPS 4: 1)

    if (tid == 0) *lds_zero = make_uint4(0, 0, 0, 0);

    // --- global -> register staging: 16 packed bytes (one K-step of one row)
    // per chunk; A has 1024 chunks per stage (2 per thread), B 512 (1) ---
    // two staging sets: the packed bytes of stage t+2 are fetched while stage t
    // is multiplied, so a fetch has two stages' time to arrive
    uint4 ra[2][2], rb[2][BCH];
    float rsa[2][NS], rsw[2][NS];

    auto load_stage = [&](int t, int set) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int c = tid + THREADS * i;
            const int row = c >> 2, s = c & 3;
            const int am = m0 + row;
            ra[set][i] = am < a.M ? *reinterpret_cast<const uint4*>(a.qa + am * rowbytes + (int64_t)t * ROWB + s * 16)
                             : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < BCH; ++i) {
            const int c = tid + THREADS * i;
            const int row = c >> 2, s = c & 3;
            const int bn = n0 + row;
            rb[set][i] = bn < a.N ? *reinterpret_cast<const uint4*>(a.qw + bn * rowbytes + (int64_t)t * ROWB + s * 16)
                                  : make_uint4(0, 0, 0, 0);
        }
        // scales: SUBS groups of this stage for BM rows of A and BN rows of B
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            const int idx = tid + THREADS * i;
            const int row = idx & (BM - 1), sub = idx / BM;
            rsa[set][i] = 0.0f;
            if (sub < SUBS && m0 + row < a.M) {
                const int k0 = t * KSTAGE + sub * a.gs;
                rsa[set][i] = a.sa[(int64_t)(m0 + row) * a.Ga + k0 / a.ga] * 0.00390625f;
            }
            const int rowb = idx & (BN - 1), subb = idx / BN;
            rsw[set][i] = 0.0f;
            if (!MIXED && subb < SUBS && n0 + rowb < a.N) {
                const int k0 = t * KSTAGE + subb * a.gs;
                rsw[set][i] = a.sw[(int64_t)(n0 + rowb) * a.Gw + k0 / a.gw];
            }
        }
    };

    // widen the staged chunks and store them: K-step s of a row occupies bytes
    // [32s, 32s+32) of the row, first half (codes 0..15) then second half
    auto store_stage = [&](int buf, int set) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int c = tid + THREADS * i;
            const int row = c >> 2, s = c & 3;
            const int o = row * LDS_STRIDE + 32 * s;
            *reinterpret_cast<uint4*>(&lds_a[buf][o]) = widen_lo(ra[set][i]);
            *reinterpret_cast<uint4*>(&lds_a[buf][o + 16]) = widen_hi(ra[set][i]);
        }
#pragma unroll
        for (int i = 0; i < BCH; ++i) {
            const int c = tid + THREADS * i;
            const int row = c >> 2, s = c & 3;
            const int o = row * LDS_STRIDE + 32 * s;
            *reinterpret_cast<uint4*>(&lds_b[buf][o]) = widen_lo(rb[set][i]);
            *reinterpret_cast<uint4*>(&lds_b[buf][o + 16]) = widen_hi(rb[set][i]);
        }
        if constexpr (SPLIT) {
            // bf16 split operands of each of the stage's SUBS groups: A row
            // (slots 0..5) x0 x0 x0 x1 x1 x2, B row y0 y1 y2 y0 y1 y0, so
            // slot k holds x_p*y_q with p+q <= 2
#pragma unroll
            for (int i = 0; i < NS; ++i) {
                const int idx = tid + THREADS * i;
                const int row = idx & (BM - 1), sub = idx / BM;
                if (sub < SUBS) {
                    uint32_t x0, x1, x2;
                    split3(rsa[set][i], x0, x1, x2);
                    spa_tab(buf, sub)[row] = make_uint4(x0 | (x0 << 16), x0 | (x1 << 16), x1 | (x2 << 16), 0);
                }
                const int rowb = idx & (BN - 1), subb = idx / BN;
                if (subb < SUBS) {
                    uint32_t y0, y1, y2;
                    split3(rsw[set][i], y0, y1, y2);
                    spb_tab(buf, subb)[rowb] = make_uint4(y0 | (y1 << 16), y2 | (y0 << 16), y1 | (y0 << 16), 0);
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < NS; ++i) {
                const int idx = tid + THREADS * i;
                const int row = idx & (BM - 1), sub = idx / BM;
                if (sub < SUBS) sa_tab(buf, sub)[row] = rsa[set][i];
                const int rowb = idx & (BN - 1), subb = idx / BN;
                if (!MIXED && subb < SUBS) sw_tab(buf, subb)[rowb] = rsw[set][i];
            }
        }
    };

    float acc[2][2][16];
    v16i P[2][2];
    v16f S11 = v16f{};   // g = 128: scale products of the last tile of the previous stage
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mt][nt][r] = 0.0f;

    // one 32x32 tile, the four K-steps of a stage
    auto mma_tile = [&](v16i& p, const v4i* fa, const v4i* fb, bool first) {
        v16i c = first ? v16i{} : p;
        c = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[0], fb[0], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[1], fb[1], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[2], fb[2], c, 0, 0, 0);
        p = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[3], fb[3], c, 0, 0, 0);
    };

    // bf16 split operands of this wave's rows and columns (lanes 32..63 read
    // the zero row: their K slots 8..15 are unused)
    v8bf opa[2], opb[2];
    auto load_split_operands = [&](int buf, int sub) {
        if constexpr (SPLIT) {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const uint4* p = (lane < 32) ? &spa_tab(buf, sub)[wm * 64 + mt * 32 + lane] : lds_zero;
                opa[mt] = __builtin_bit_cast(v8bf, *p);
            }
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const uint4* p = (lane < 32) ? &spb_tab(buf, sub)[wn * 64 + nt * 32 + lane] : lds_zero;
                opb[nt] = __builtin_bit_cast(v8bf, *p);
            }
        }
    };

    // The 16 scale products S = s_a[m]*s_w[n] (or s_a[m] alone in mixed mode)
    // of tile (mt, nt) in accumulator layout, for a group of >= 128 held in
    // stage buffer `buf`.
    auto tile_scales = [&](int buf, int mt, int nt) -> v16f {
        if constexpr (SPLIT) {
            const uint4* pa = (lane < 32) ? &spa_tab(buf, 0)[wm * 64 + mt * 32 + lane] : lds_zero;
            const uint4* pb = (lane < 32) ? &spb_tab(buf, 0)[wn * 64 + nt * 32 + lane] : lds_zero;
            return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, *pa),
                                                           __builtin_bit_cast(v8bf, *pb), v16f{}, 0, 0, 0);
        } else {
            v16f S;
            const float* sp = sa_tab(buf, 0) + wm * 64 + mt * 32 + 4 * (lane >> 5);
            const float sw = MIXED ? 1.0f : sw_tab(buf, 0)[wn * 64 + nt * 32 + (lane & 31)];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 v = *reinterpret_cast<const float4*>(sp + 8 * q);
                S[4 * q + 0] = MIXED ? v.x : v.x * sw;
                S[4 * q + 1] = MIXED ? v.y : v.y * sw;
                S[4 * q + 2] = MIXED ? v.z : v.z * sw;
                S[4 * q + 3] = MIXED ? v.w : v.w * sw;
            }
            return S;
        }
    };

    // MFMAs of one tile (a new group: zero start), each followed by the rescale
    // of 4 outputs of finished tile (rm, rn) with scale products S; the fences
    // keep this issue order.
    auto mma_tile_rescaling = [&](v16i& p, const v4i* fa, const v4i* fb, int rm, int rn, const v16f& S) {
        v16i c = v16i{};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            c = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[s], fb[s], c, 0, 0, 0);
#pragma unroll
            for (int r = 4 * s; r < 4 * s + 4; ++r) {
                acc[rm][rn][r] = fmaf(S[r], (float)P[rm][rn][r], acc[rm][rn][r]);
                // anchors the update here (code motion before scheduling would
                // otherwise gather all updates after the last MFMA)
                asm volatile("" : "+v"(acc[rm][rn][r]));
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        p = c;
    };

    auto debug_tile = [&](int mt, int nt, int j) {
        if (DEBUG_P) {
            const int n = n0 + wn * 64 + nt * 32 + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm * 64 + mt * 32 + acc_row(r, lane);
                if (m < a.M && n < a.N)
                    if (int32_t* d = psum_at(a.psum, a.prows, m, n, a.N, a.G, j)) *d = P[mt][nt][r] >> 8;
            }
        }
    };

    // Rescale the finished group held in P[mt][nt] into acc[mt][nt] (scale
    // group `sub` of stage buffer `buf`; global group index j).
    auto rescale_tile_sub = [&](int buf, int sub, int mt, int nt, int j) {
        if constexpr (SPLIT) {
            // S = s_a (x) s_w for the tile, on the matrix unit
            const v16f S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opa[mt], opb[nt], v16f{}, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mt][nt][r] = fmaf(S[r], (float)P[mt][nt][r], acc[mt][nt][r]);
        } else {
            const float* sp = sa_tab(buf, sub) + wm * 64 + mt * 32 + 4 * (lane >> 5);
            float sw = 1.0f;
            if (!MIXED) sw = sw_tab(buf, sub)[wn * 64 + nt * 32 + (lane & 31)];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 v = *reinterpret_cast<const float4*>(sp + 8 * q);
                const float sa[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 4 * q + i;
                    const float S = MIXED ? sa[i] : sa[i] * sw;
                    acc[mt][nt][r] = fmaf(S, (float)P[mt][nt][r], acc[mt][nt][r]);
                }
            }
        }
        debug_tile(mt, nt, j);
    };
    auto rescale_tile = [&](int buf, int mt, int nt, int j) { rescale_tile_sub(buf, 0, mt, nt, j); };
    auto rescale_all = [&](int buf, int sub, int j) {
        if constexpr (SPLIT) load_split_operands(buf, sub);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) rescale_tile_sub(buf, sub, mt, nt, j);
    };

    load_stage(0, 0);
    if (stages > 1) load_stage(1, 1);
    store_stage(0, 0);
    __syncthreads();

    // stage t uses LDS buffer t&1 and staging set t&1; the loop is unrolled by
    // two so that both indices are compile-time constants
    for (int t0 = 0; t0 < stages; t0 += 2)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int t = t0 + h;
        if (t >= stages) break;
        const int buf = h;
        if (t + 2 < stages) load_stage(t + 2, h);

        const uint8_t* la = lds_a[buf] + (wm * 64 + (lane & 31)) * LDS_STRIDE + 16 * (lane >> 5);
        const uint8_t* lb = lds_b[buf] + (wn * 64 + (lane & 31)) * LDS_STRIDE + 16 * (lane >> 5);
        if constexpr (SMALL) {
            // groups of 32 / 64: step-major, a rescale after every group; the
            // loop stays rolled so only one step's fragments are live across it
#pragma unroll 1
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
                if (s % GS_STEPS == 0) {
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                        for (int nt = 0; nt < 2; ++nt)
                            P[mt][nt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[mt], fb[nt], v16i{}, 0, 0, 0);
                } else {
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                        for (int nt = 0; nt < 2; ++nt)
                            P[mt][nt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[mt], fb[nt], P[mt][nt], 0, 0, 0);
                }
                if (GS_STEPS == 1) rescale_all(buf, s, t * MAX_SUB + s);
                if (GS_STEPS == 2 && (s & 1)) rescale_all(buf, s >> 1, t * (MAX_SUB / 2) + (s >> 1));
            }
        } else if constexpr (GS_STEPS == 4) {
            // One group per stage (g = 128), explicit issue order.  Each tile's
            // four MFMAs are each followed by 8 vector instructions of the
            // rescale of the tile finished before it (4 of its 16 outputs:
            // convert + fma), which run on the vector ALU while the MFMA
            // computes.  The last tile of a stage is rescaled during the first
            // tile of the next stage, from scale products kept in registers
            // (P[1][1] is only overwritten by the last tile).
            const int j = t;
            v4i fa[4], fb0[4], fb1[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                fa[s] = *reinterpret_cast<const v4i*>(la + 32 * s);
                fb0[s] = *reinterpret_cast<const v4i*>(lb + 32 * s);
            }
            if (t > 0) {
                mma_tile_rescaling(P[0][0], fa, fb0, 1, 1, S11);
                debug_tile(1, 1, j - 1);
            } else {
                mma_tile(P[0][0], fa, fb0, true);
            }
            v16f Sx = tile_scales(buf, 0, 0);
#pragma unroll
            for (int s = 0; s < 4; ++s) fb1[s] = *reinterpret_cast<const v4i*>(lb + 32 * LDS_STRIDE + 32 * s);
            mma_tile_rescaling(P[0][1], fa, fb1, 0, 0, Sx);
            debug_tile(0, 0, j);
            Sx = tile_scales(buf, 0, 1);
            // the first B fragment is read again rather than kept live: three
            // tiles' fragments at once do not fit next to the accumulators
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                fa[s] = *reinterpret_cast<const v4i*>(la + 32 * LDS_STRIDE + 32 * s);
                fb0[s] = *reinterpret_cast<const v4i*>(lb + 32 * s);
            }
            mma_tile_rescaling(P[1][0], fa, fb0, 0, 1, Sx);
            debug_tile(0, 1, j);
            Sx = tile_scales(buf, 1, 0);
            mma_tile_rescaling(P[1][1], fa, fb1, 1, 0, Sx);
            debug_tile(1, 0, j);
            S11 = tile_scales(buf, 1, 1);
        } else {
            // groups spanning several stages (g >= 256): tile-major; the
            // rescale comes once every stages_per_group stages
            const bool first = t % stages_per_group == 0;
            const bool last = (t + 1) % stages_per_group == 0;
            const int j = t / stages_per_group;
            v4i fa[4], fb0[4], fb1[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                fa[s] = *reinterpret_cast<const v4i*>(la + 32 * s);
                fb0[s] = *reinterpret_cast<const v4i*>(lb + 32 * s);
            }
            mma_tile(P[0][0], fa, fb0, first);
#pragma unroll
            for (int s = 0; s < 4; ++s) fb1[s] = *reinterpret_cast<const v4i*>(lb + 32 * LDS_STRIDE + 32 * s);
            mma_tile(P[0][1], fa, fb1, first);
#pragma unroll
            for (int s = 0; s < 4; ++s) fa[s] = *reinterpret_cast<const v4i*>(la + 32 * LDS_STRIDE + 32 * s);
            mma_tile(P[1][0], fa, fb0, first);
            mma_tile(P[1][1], fa, fb1, first);
            if (last) {
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) {
                        const v16f S = tile_scales(buf, mt, nt);
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            acc[mt][nt][r] = fmaf(S[r], (float)P[mt][nt][r], acc[mt][nt][r]);
                        debug_tile(mt, nt, j);
                    }
            }
        }

        if (t + 1 < stages) store_stage(buf ^ 1, h ^ 1);
        __syncthreads();
    }

    if constexpr (GS_STEPS == 4) {
        // the last stage's tile (1,1)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[1][1][r] = fmaf(S11[r], (float)P[1][1][r], acc[1][1][r]);
        debug_tile(1, 1, stages - 1);
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
        if (dbg) gemm_tiled_kernel<GS_STEPS, true, true><<<grid, THREADS, 0, stream>>>(t);
        else gemm_tiled_kernel<GS_STEPS, true, false><<<grid, THREADS, 0, stream>>>(t);
    } else {
        if (dbg) gemm_tiled_kernel<GS_STEPS, false, true><<<grid, THREADS, 0, stream>>>(t);
        else gemm_tiled_kernel<GS_STEPS, false, false><<<grid, THREADS, 0, stream>>>(t);
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
    t.prows = p.prows;
    const bool mixed = (p.gw == p.K) && (p.ga != p.gw);
    if (t.gs == 32)
        launch_tiled_mode<1>(t, mixed, stream);
    else if (t.gs == 64)
        launch_tiled_mode<2>(t, mixed, stream);
    else if (t.gs == KSTAGE)
        launch_tiled_mode<4>(t, mixed, stream);
    else
        launch_tiled_mode<0>(t, mixed, stream);
    return hipGetLastError();
}

}  // namespace apex4
