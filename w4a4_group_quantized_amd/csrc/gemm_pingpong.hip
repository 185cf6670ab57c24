// W4A4 GEMM with per-group dequantization on gfx950: the ping-pong tiled
// kernel for compute-bound calls with groups of 32, 64, 128 or 256 (or one
// group over K).
//
// The computation is the APEX4 page's (Abstract): INT4 x INT4 products summed
// exactly per K-group on the matrix units, every group's integer sum rescaled
// by s_a*s_w and accumulated in fp32 on the vector ALUs.  Per 32x32 tile and
// group of 128 the int8 MFMA is busy 128 cycles and the rescale (convert +
// fma for 16 outputs per lane) keeps the vector ALU busy about as long, so
// the two must run at the same time to get near the matrix-unit bound.
//
// Ping-pong.  A workgroup of 8 waves computes a 256x128 tile of Y, each wave a
// 64x64 sub-tile (2x2 MFMA tiles of 32x32x32 int8).  Waves are placed on the
// four SIMDs of a CU round-robin, so SIMD i holds waves i and i+4.  Waves 0..3
// run half a K-stage ahead of waves 4..7: between two barriers one wave of
// every SIMD issues the matrix work of a stage while the other issues the
// vector rescale of the stage it finished before; at the next barrier the
// roles swap.  The hardware then keeps both units of the SIMD busy from two
// instruction streams, which no static schedule of one wave achieved here.
//
//   waves 0..3, stage t:  | matrix(t)    | rescale(t)  |
//   waves 4..7, stage t:  | rescale(t-1) | matrix(t)   |
//
// The matrix phase holds the fragment reads and the 16 int8 MFMAs of the
// stage, most of the copy of stage t+1 (16-byte global loads two stages
// ahead, widened to int8 and stored to LDS), and the scale products
// S = s_a * s_w of the 4 tiles.  The vector phase is the convert + fma of
// the 64 outputs per lane, from registers, and the last of the thread's
// three copy chunks (the matrix phase is the longer one; in mixed mode, with
// its larger rescale, the whole copy stays in the matrix phase).
//
// LDS: A and B stages (int8, widened from nibbles in the global -> LDS copy,
// 144-byte rows so that 16 consecutive rows hit every bank once) and the
// scale operands are double-buffered.
//
// Nibble widening, the 2^-8 fold, the bf16 split of the scale products and
// the fixed-order fp32 accumulation are those of the other tiled kernel:
// (w << 4) & 0xF0F0F0F0 and w & 0xF0F0F0F0 give the int8 values 16*c, the
// MFMA returns 256*P exactly, and S = (2^-8 s_a) * s_w comes from one bf16
// MFMA over the exact three-piece splits of both scales (six of the nine cross
// products; the three dropped are below 2^-23 of S).  One group over all of K
// (per-channel scales) keeps P in the MFMA accumulator through the loop and
// is rescaled once; with no rescale to overlap, both wave groups then run the
// matrix work of every stage together (one barrier per stage: the ping-pong
// offset would only leave each SIMD's matrix unit with one wave).  Mixed mode (per-channel weight scales, activation groups
// of 64, 128 or 256) rescales with s_a alone and applies s_w in the epilogue.
//
// Groups of 64 and 32.  A 128-value stage holds two (four) groups, so the
// ping-pong runs per group: four (eight) phases per stage, in each a wave
// either issues one group's 8 (4) MFMAs and its scale products, or rescales
// the group it finished before.  The copy of the next stage is stored in the
// stage's matrix phases, and its scale rows hold every group of the stage
// (156 KB of LDS in all).  Several groups' int32 sums would not fit in the
// registers beside the accumulators; one group per phase needs no more than
// groups of 128 do.  At groups of 32 the four groups' scale rows fit in LDS
// only as single 16-byte entries: their products come from the K = 8
// split-operand MFMA (v_mfma_f32_32x32x8_bf16), which takes slots 0..3 from
// lanes 0..31 and 4..7 from lanes 32..63, so no zero half is stored.
//
// FP8-coded operands (apex4_gemm_w4a4_f8).  The same kernel with each code
// stored as its exact E4M3 byte: the copy stores the bytes as they come (no
// widening), a 128-code stage is two K-steps of
// v_mfma_scale_f32_32x32x64_f8f6f4 (unit block scales), whose fp32 result is
// the exact group sum, so the rescale is one fma per output; no 2^-8 fold.
//
// Rounds of tiles.  One workgroup fills a CU, so a launch runs in rounds of
// one tile per CU.  A last round that would leave more than half the CUs
// idle (e.g. 96 of 256, or a call with only a few tiles) is run as 2 to 4
// parts of K instead (groups of one stage, split at group boundaries) on as
// many times the workgroups; their fp32 tile sums go to the caller's
// workspace and a small kernel adds the parts in a fixed order and writes Y
// as the epilogue does.
#include "internal.h"

#include <atomic>
#include <type_traits>

namespace apex4 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 256;
constexpr int BN = 128;
constexpr int THREADS = 512;
constexpr int HALF = THREADS / 2;       // threads per wave group
constexpr int KSTAGE = 128;             // K values per stage
constexpr int ROWB = KSTAGE / 2;        // packed bytes per row per stage
constexpr int STRIDE = 144;             // LDS bytes per int8 row (128 + 16 padding)
constexpr uint32_t A_BYTES = BM * STRIDE;
constexpr uint32_t B_BYTES = BN * STRIDE;

struct PPArgs {
    const uint8_t* qa;
    const float* sa;
    const uint8_t* qw;
    const float* sw;
    int M, N, K;
    int Ga, Gw;        // scale columns per row: K/ga, K/gw
    int spg;           // stages per group: gs / 128 (1, 2, or all of K; -1: groups of 64, -2: of 32)
    int G;             // K / gs
    _Float16* y16;
    float* y32;
    int32_t* psum;
    PsumRows prows;
    // Tiles: BM x BN blocks of Y, numbered in bands of group_m row blocks:
    // down a column of the band, then the next column, so that the
    // workgroups in flight share few A and B blocks.  The chip deals
    // workgroup b to XCD b mod 8, each XCD with its own L2, so in a full-K
    // launch of B workgroups, b (< 8 floor(B/8)) takes tile tile0 +
    // (b mod 8) floor(B/8) + b div 8: each XCD walks a contiguous range of
    // tile ids, its 32 workgroups in flight covering 4 row blocks x 8 column
    // blocks (the epilogue writes Y); in a K-split launch (part != null), tile tile0 + b % ntail
    // over K part q = b / ntail of nparts (stages [q S / nparts, (q+1) S /
    // nparts) of the S = K/128), writing its fp32 sums to part[q][b % ntail]
    // ([BM][BN], before s_w in mixed mode) for the reduction kernel.
    int tiles_n;       // tiles along N: ceil(N / BN)
    int tiles_m;       // tiles along M: ceil(M / BM)
    int group_m;       // row blocks per band of the tile order
    int tile0;
    int ntail;
    int nparts;
    float* part;
};

__device__ inline __amdgpu_buffer_rsrc_t buffer_of(const void* p, uint32_t bytes)
{
    // raw buffer: loads past `bytes` return zeros
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

__device__ inline uint4 widen_lo(uint4 w)
{
    return make_uint4((w.x << 4) & 0xF0F0F0F0u, w.x & 0xF0F0F0F0u,
                      (w.y << 4) & 0xF0F0F0F0u, w.y & 0xF0F0F0F0u);
}

__device__ inline uint4 widen_hi(uint4 w)
{
    return make_uint4((w.z << 4) & 0xF0F0F0F0u, w.z & 0xF0F0F0F0u,
                      (w.w << 4) & 0xF0F0F0F0u, w.w & 0xF0F0F0F0u);
}

__device__ inline uint32_t bf16_trunc_bits(float x) { return __builtin_bit_cast(uint32_t, x) >> 16; }

// exact split s = x0 + x1 + x2 into bf16 values (truncation at each step)
__device__ inline void split3(float s, uint32_t& x0, uint32_t& x1, uint32_t& x2)
{
    x0 = bf16_trunc_bits(s);
    const float r1 = s - __builtin_bit_cast(float, x0 << 16);
    x1 = bf16_trunc_bits(r1);
    const float r2 = r1 - __builtin_bit_cast(float, x1 << 16);
    x2 = bf16_trunc_bits(r2);
}

// (row block, column block) of a tile id: bands of group_m row blocks, each
// walked column by column
__device__ inline void tile_coords(const PPArgs& a, int tile, int& by, int& bx)
{
    const int band = a.group_m * a.tiles_n;
    const int g = tile / band;
    const int first = g * a.group_m;
    const int rows = min(a.group_m, a.tiles_m - first);
    const int local = tile - g * band;
    by = first + local % rows;
    bx = local / rows;
}

// Register anchors.  An empty volatile asm that takes a value in and out keeps
// its producers before and its consumers after this point in program order;
// volatile asm statements and the barrier keep their relative order.  The
// arithmetic of each phase stays between its two barriers this way (pure
// register arithmetic may otherwise be moved across a barrier).
__device__ inline void anchor(float& x) { asm volatile("" : "+v"(x)); }
__device__ inline void anchor(int& x) { asm volatile("" : "+v"(x)); }
__device__ inline void anchor(uint4& x)
{
    asm volatile("" : "+v"(x.x));
    asm volatile("" : "+v"(x.y));
    asm volatile("" : "+v"(x.z));
    asm volatile("" : "+v"(x.w));
}

__device__ inline int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// LDS of one workgroup (NG: groups per stage, 2 for groups of 64, 4 for
// groups of 32; HV: 16-byte halves per scale entry, 1 where the scale
// products use the K = 8 split-operand MFMA, which needs no zero half)
template <int NG, int HV>
struct PPShared {
    uint8_t a[2][A_BYTES];
    uint8_t b[2][B_BYTES];
    // Scale operands, per stage buffer and group: two 16-byte halves per tile row, half
    // 0 holding the bf16 pieces in slots 0..5 and zeros in 6..7, half 1 zeros
    // (lanes 32..63 of the split-operand MFMA read it); stored half-major, so
    // that 8 consecutive rows' reads of one half are 128 contiguous bytes (as
    // 32-byte rows they were 2-way bank conflicted).  In mixed mode ta holds
    // fp32 2^-8 s_a in its first BM dwords.
    uint4 ta[2][NG][HV][BM];
    uint4 tb[2][NG][HV][BN];
};

// groups per stage and scale-row halves of a stages-per-group mode
template <int SPG> struct PPMode {
    static constexpr int NG = SPG == -2 ? 4 : SPG == -1 ? 2 : 1;
    static constexpr int HV = SPG == -2 ? 1 : 2;
};

// Orders this wave's LDS accesses around the workgroup barrier (LDS only:
// global loads in flight stay in flight).
// The scheduling fences keep every instruction on its side of the barrier.
__device__ inline void lds_barrier()
{
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    __builtin_amdgcn_sched_barrier(0);
}

// SPG: stages per group, 1 (g = 128), 2 (g = 256) or 0 (one group, g = K);
// -1: groups of 64, two per stage; -2: groups of 32, four per stage (GN below).
// EARLY: this wave belongs to waves 0..3.
// F8: FP8-coded operands (one byte per code, the codes' exact E4M3 values):
// a stage of 128 codes is 128 bytes per row, copied in 6 chunks per thread
// through one register set (stored before the next stage's loads are
// issued), two 64-code K-steps of the FP8 MFMA.
template <bool MIXED, bool DEBUG_P, int SPG, bool EARLY, bool F8>
__device__ __forceinline__ void pp_body(const PPArgs& a, PPShared<PPMode<SPG>::NG, PPMode<SPG>::HV>& sh)
{
    constexpr bool GN = SPG < 0;                 // groups of 64 or 32: several per stage
    constexpr int NG = PPMode<SPG>::NG;          // groups per stage
    constexpr int HV = PPMode<SPG>::HV;          // scale-row halves in sh.ta, sh.tb
    constexpr int KST = KSTAGE;                  // K values per stage
    constexpr int ROWB_S = F8 ? 128 : ROWB;      // operand bytes per row per stage
    constexpr int CPR = ROWB_S / 16;             // 16-byte chunks per row per stage
    constexpr int NCH = 3 * CPR / 4;             // chunks per thread per stage
    constexpr int SPLIT = MIXED ? NCH : NCH - 1;  // chunks stored in the matrix phase (groups of one stage)
    constexpr int NSET = F8 ? 1 : 2;             // register sets of the copy
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;      // 64-row, 64-column sub-tile
    int lin = blockIdx.x, kpart = 0;
    if (a.part) {
        kpart = lin / a.ntail;
        lin -= kpart * a.ntail;
    } else {
        // XCD-aware order: XCD b mod 8 takes a contiguous range of tile ids
        const int per = (int)gridDim.x >> 3;
        if (lin < per * 8) lin = (lin & 7) * per + (lin >> 3);
    }
    const int tile = a.tile0 + lin;
    int by, bx;
    tile_coords(a, tile, by, bx);
    const int m0 = by * BM, n0 = bx * BN;
    const uint32_t rowbytes = F8 ? (uint32_t)a.K : (uint32_t)a.K / 2;
    // this workgroup's stages: s0 .. s0 + stages - 1
    const int all_stages = a.K / KST;
    const int s0 = a.part ? kpart * all_stages / a.nparts : 0;
    const int stages = a.part ? (kpart + 1) * all_stages / a.nparts - s0 : all_stages;
    const int rows_a = min(BM, a.M - m0), rows_b = min(BN, a.N - n0);
    // Per-workgroup buffers: rows past M (N) lie past the end and read zeros.
    // The per-stage offset goes into the scalar offset of the load.
    const __amdgpu_buffer_rsrc_t rA = buffer_of(a.qa + (int64_t)m0 * rowbytes, (uint32_t)rows_a * rowbytes);
    const __amdgpu_buffer_rsrc_t rB = buffer_of(a.qw + (int64_t)n0 * rowbytes, (uint32_t)rows_b * rowbytes);
    const __amdgpu_buffer_rsrc_t rSA = buffer_of(a.sa + (int64_t)m0 * a.Ga, (uint32_t)rows_a * a.Ga * 4);
    const __amdgpu_buffer_rsrc_t rSW = buffer_of(a.sw + (int64_t)n0 * a.Gw, (uint32_t)rows_b * a.Gw * 4);

    // --- this thread's share of a stage copy: NCH chunks of 16 bytes (3 of
    // packed codes, one 32-code K-step of a row each; FP8: 6 of 16 codes).
    // Waves 0..3: A rows 0..191 and the A scales; waves 4..7: A rows
    // 192..255, all of B and the B scales. ---
    const int ht = EARLY ? tid : tid - HALF;
    uint32_t goff[NCH], loff[NCH];
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        int c;
        if (EARLY) c = ht + HALF * j;                                  // A rows 0..191
        else c = j < CPR / 4 ? 192 * CPR + ht + HALF * j : ht + HALF * (j - CPR / 4);   // A 192..255; B
        const int row = (unsigned)c / CPR, s = (unsigned)c % CPR;
        goff[j] = (uint32_t)row * rowbytes + 16 * s;
        loff[j] = row * STRIDE + (F8 ? 16 : 32) * s;
    }
    // chunk j's operand: A, or B for the chunks past the first CPR/4 of waves 4..7
    auto chunk_is_b = [](int j) { return !EARLY && j >= CPR / 4; };
    const bool has_scale = EARLY ? true : (!MIXED && ht < BN);
    // threads without a scale row load from past the end (zeros), so that
    // every load is unconditional and the wait counts stay exact
    const uint32_t soff = !has_scale ? 0x80000000u : EARLY ? (uint32_t)ht * a.Ga * 4 : (uint32_t)ht * a.Gw * 4;

    uint4 rq[NSET][NCH];
    float rs[NSET][NG];
    auto load_stage = [&](int t, int set) {
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            const u32x4 v =
                __builtin_amdgcn_raw_buffer_load_b128(chunk_is_b(j) ? rB : rA, (int)goff[j], (s0 + t) * ROWB_S, 0);
            rq[set][j] = make_uint4(v.x, v.y, v.z, v.w);
        }
        // the scale of the group (groups of 64 or 32: the groups) that stage t
        // belongs to (several groups per stage: stages past the end load the
        // last stage's scales, which are not used)
        const int g = (SPG == 1 ? s0 + t : SPG == 2 ? (s0 + t) >> 1 : GN ? NG * min(s0 + t, all_stages - 1) : 0) * 4;
        if (EARLY || !MIXED)
#pragma unroll
            for (int q = 0; q < NG; ++q)
                rs[set][q] = __builtin_bit_cast(
                    float, __builtin_amdgcn_raw_buffer_load_b32(EARLY ? rSA : rSW, (int)soff, g + 4 * q, 0));
    };
    // the scale rows of groups q0 .. q1-1 of a stage (register set `set`)
    // into stage buffer `buf`
    auto store_scales = [&](int buf, int set, int q0, int q1) {
#pragma unroll
        for (int q = 0; q < NG; ++q) {
            if (q < q0 || q >= q1) continue;
            if (EARLY) {
                // A scale of row ht, with the 2^-8 of the widened operands folded
                // in (FP8 codes are the values themselves)
                const float s = F8 ? rs[set][q] : rs[set][q] * 0.00390625f;
                if (MIXED) {
                    reinterpret_cast<float*>(sh.ta[buf][q])[ht] = s;
                } else {
                    uint32_t x0, x1, x2;
                    split3(s, x0, x1, x2);
                    // slots 0..5: x0 x0 x0 x1 x1 x2 (paired with y0 y1 y2 y0 y1 y0)
                    sh.ta[buf][q][0][ht] = make_uint4(x0 | (x0 << 16), x0 | (x1 << 16), x1 | (x2 << 16), 0);
                }
            } else if (has_scale) {
                uint32_t y0, y1, y2;
                split3(rs[set][q], y0, y1, y2);
                sh.tb[buf][q][0][ht] = make_uint4(y0 | (y1 << 16), y2 | (y0 << 16), y1 | (y0 << 16), 0);
            }
        }
    };
    // (chunks j0 .. j1-1 of the thread's share, default all of them, and the
    // scale row if `scale`)
    auto store_stage = [&](int buf, int set, int j0 = 0, int j1 = 1 << 30, bool scale = true) {
#pragma unroll
        for (int j = 0; j < NCH; ++j)
            if (j >= j0 && j < j1) anchor(rq[set][j]);   // widen in this phase
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            if (j < j0 || j >= j1) continue;
            uint8_t* base = chunk_is_b(j) ? sh.b[buf] : sh.a[buf];
            if (F8) {
                *reinterpret_cast<uint4*>(base + loff[j]) = rq[set][j];
            } else {
                *reinterpret_cast<uint4*>(base + loff[j]) = widen_lo(rq[set][j]);
                *reinterpret_cast<uint4*>(base + loff[j] + 16) = widen_hi(rq[set][j]);
            }
        }
        if (scale) store_scales(buf, set, 0, NG);
    };

    float acc[2][2][16];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mt][nt][r] = 0.0f;
    using PT = typename std::conditional<F8, v16f, v16i>::type;
    PT P[2][2];
    v16f S[2][2];   // scale products of the group in P
    if (SPG == 0) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) P[mt][nt] = PT{};
    }

    // fragment bases: row lane & 31 of the wave's tiles, K bytes from 16 (or,
    // FP8, 32) * (lane >> 5)
    const uint32_t frag = (wm * 64 + (lane & 31)) * STRIDE + (F8 ? 32 : 16) * (lane >> 5);
    const uint32_t fragb = (wn * 64 + (lane & 31)) * STRIDE + (F8 ? 32 : 16) * (lane >> 5);
    const int trow = lane & 31, thalf = lane >> 5;
    // The scale products S of the 4 tiles for group q of stage buffer `buf`,
    // on the matrix unit, so that the vector phase has no LDS or matrix-unit
    // dependency.
    auto scale_products = [&](int buf, int q = 0) {
        if (MIXED) {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const float* sp = reinterpret_cast<const float*>(sh.ta[buf][q]) + wm * 64 + mt * 32 + 4 * thalf;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float4 v = *reinterpret_cast<const float4*>(sp + 8 * u);
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) {
                        S[mt][nt][4 * u + 0] = v.x;
                        S[mt][nt][4 * u + 1] = v.y;
                        S[mt][nt][4 * u + 2] = v.z;
                        S[mt][nt][4 * u + 3] = v.w;
                    }
                }
            }
        } else {
            v8bf opa[2], opb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                if constexpr (HV == 2) {
                    opa[i] = __builtin_bit_cast(v8bf, sh.ta[buf][q][thalf][wm * 64 + i * 32 + trow]);
                    opb[i] = __builtin_bit_cast(v8bf, sh.tb[buf][q][thalf][wn * 64 + i * 32 + trow]);
                }
            }
            if constexpr (HV == 2) {
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt)
                        S[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opa[mt], opb[nt], v16f{}, 0, 0, 0);
            } else {
                // one 16-byte entry per scale: the K = 8 split-operand MFMA,
                // lanes 0..31 taking slots 0..3 and lanes 32..63 slots 4..7
                // (two of them zero), so no zero half is needed
                v4s oa[2], ob[2];
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    oa[i] = __builtin_bit_cast(
                        v4s, reinterpret_cast<const uint2*>(&sh.ta[buf][q][0][wm * 64 + i * 32 + trow])[thalf]);
                    ob[i] = __builtin_bit_cast(
                        v4s, reinterpret_cast<const uint2*>(&sh.tb[buf][q][0][wn * 64 + i * 32 + trow])[thalf]);
                }
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt)
                        S[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(oa[mt], ob[nt], v16f{}, 0, 0, 0);
            }
        }
    };
    // Matrix phase of stage buffer `buf`: the 16 int8 MFMAs, K-step-major so
    // that consecutive MFMAs are independent (`zero`: the stage starts a group
    // and the MFMAs start from zero), then, when the stage ends a group
    // (`ends`), the scale products.
    auto mma_stage = [&](int buf, bool zero, bool ends) {
        const uint8_t* la = sh.a[buf] + frag;
        const uint8_t* lb = sh.b[buf] + fragb;
        if constexpr (F8) {
            // two K-steps of 64: 32 bytes per lane and tile each, 8 MFMAs
            // (the stage is one group: P starts from zero)
            v8i ga[2][2], gb[2][2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const v4i a0 = *reinterpret_cast<const v4i*>(la + i * 32 * STRIDE + 64 * ks);
                    const v4i a1 = *reinterpret_cast<const v4i*>(la + i * 32 * STRIDE + 64 * ks + 16);
                    const v4i b0 = *reinterpret_cast<const v4i*>(lb + i * 32 * STRIDE + 64 * ks);
                    const v4i b1 = *reinterpret_cast<const v4i*>(lb + i * 32 * STRIDE + 64 * ks + 16);
                    ga[i][ks] = v8i{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
                    gb[i][ks] = v8i{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
                }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt)
                        P[mt][nt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            ga[mt][ks], gb[nt][ks], ks == 0 ? v16f{} : P[mt][nt], 0, 0, 0, 127, 0, 127);
            if (ends) scale_products(buf);
            return;
        }
        v4i fa[2][4], fb[2][4];
        // one group over K: P is live across stages but nothing else is, so
        // the fragments can all be read first as well
        const bool upfront = zero || SPG == 0;
        if (upfront) {
            // all fragments first
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    fa[i][s] = *reinterpret_cast<const v4i*>(la + i * 32 * STRIDE + 32 * s);
                    fb[i][s] = *reinterpret_cast<const v4i*>(lb + i * 32 * STRIDE + 32 * s);
                }
            // (one group: every read issued before the first MFMA)
            if (SPG == 0) __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if (!upfront) {
                // P is live from the stage before (groups of two stages): the
                // fragments K-step by K-step (kept apart by scheduling
                // barriers), fewer registers at once
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    fa[i][s] = *reinterpret_cast<const v4i*>(la + i * 32 * STRIDE + 32 * s);
                    fb[i][s] = *reinterpret_cast<const v4i*>(lb + i * 32 * STRIDE + 32 * s);
                }
            }
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
                    P[mt][nt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[mt][s], fb[nt][s],
                                                                      (zero && s == 0) ? v16i{} : P[mt][nt], 0, 0, 0);
        }
        if (ends) scale_products(buf);
    };
    // Several groups per stage: the matrix phase of group q of stage buffer
    // `buf`, its K-steps (groups of 64: 2q and 2q+1, 8 MFMAs; groups of 32:
    // q, 4 MFMAs) from zero, then its scale products.
    auto mma_group = [&](int buf, int q) {
        constexpr int KS = 4 / NG;   // 32-value K-steps per group
        const uint8_t* la = sh.a[buf] + frag + 32 * KS * q;
        const uint8_t* lb = sh.b[buf] + fragb + 32 * KS * q;
        if constexpr (F8) {
            // FP8 operands, groups of 64: one 64-value K-step of the FP8 MFMA
            // per tile (32 bytes per lane), whose fp32 result is the group sum
            v8i ga[2], gb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const v4i a0 = *reinterpret_cast<const v4i*>(la + i * 32 * STRIDE);
                const v4i a1 = *reinterpret_cast<const v4i*>(la + i * 32 * STRIDE + 16);
                const v4i b0 = *reinterpret_cast<const v4i*>(lb + i * 32 * STRIDE);
                const v4i b1 = *reinterpret_cast<const v4i*>(lb + i * 32 * STRIDE + 16);
                ga[i] = v8i{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
                gb[i] = v8i{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
            }
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
                    P[mt][nt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ga[mt], gb[nt], v16f{}, 0, 0, 0, 127,
                                                                                0, 127);
            scale_products(buf, q);
            return;
        }
        v4i fa[2][KS], fb[2][KS];
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                fa[i][s] = *reinterpret_cast<const v4i*>(la + i * 32 * STRIDE + 32 * s);
                fb[i][s] = *reinterpret_cast<const v4i*>(lb + i * 32 * STRIDE + 32 * s);
            }
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
                    P[mt][nt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[mt][s], fb[nt][s],
                                                                      s == 0 ? v16i{} : P[mt][nt], 0, 0, 0);
        scale_products(buf, q);
    };

    // Vector phase: acc += S (.) P for the finished group j (counted from
    // this workgroup's first stage s0; the debug sums take the index over all
    // of K).  The anchors keep the conversion and the updates between this
    // phase's barriers.
    auto rescale = [&](int j) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    auto x = P[mt][nt][r];
                    anchor(x);
                    P[mt][nt][r] = x;
                    float y = S[mt][nt][r];
                    anchor(y);
                    S[mt][nt][r] = y;
                }
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc[mt][nt][r] = fmaf(S[mt][nt][r], (float)P[mt][nt][r], acc[mt][nt][r]);
                if (DEBUG_P) {
                    const int n = n0 + wn * 64 + nt * 32 + (lane & 31);
                    const int jg = SPG == 0 ? j : GN ? NG * s0 + j : s0 / SPG + j;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int m = m0 + wm * 64 + mt * 32 + acc_row(r, lane);
                        if (m < a.M && n < a.N)
                            if (int32_t* d = psum_at(a.psum, a.prows, m, n, a.N, a.G, jg))
                                *d = F8 ? (int)P[mt][nt][r] : (int)P[mt][nt][r] >> 8;
                    }
                }
            }
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int r = 0; r < 16; ++r) anchor(acc[mt][nt][r]);
    };

    // --- prologue: the zero halves of the scale rows, stages 0 and 1 in
    // flight, stage 0 into buffer 0 ---
    if (!MIXED) {
        if constexpr (HV == 2) {
#pragma unroll
            for (int q = 0; q < NG; ++q)
                for (int i = tid; i < 2 * (BM + BN); i += THREADS) {
                    if (i < 2 * BM) sh.ta[i / BM][q][HV - 1][i % BM] = make_uint4(0, 0, 0, 0);
                    else sh.tb[(i - 2 * BM) / BN][q][HV - 1][(i - 2 * BM) % BN] = make_uint4(0, 0, 0, 0);
                }
        }
    }
    if constexpr (F8) {
        load_stage(0, 0);
        store_stage(0, 0);
        load_stage(1, 0);
    } else {
        load_stage(0, 0);
        load_stage(1, 1);
        store_stage(0, 0);
    }
    lds_barrier();

    // Stage t uses A/B and scale buffer t&1 and register set t&1; the loop is
    // unrolled by two so that these are compile-time indices.
    if constexpr (NG == 4) {
        // Groups of 32: per wave, each group's matrix work followed by the
        // rescale of the group before, the late waves one group behind the
        // early ones, with one barrier per stage: the copy of stage t+1 goes
        // to the buffer that every wave finished reading before the last
        // barrier, and is read only after the next one, so the barriers
        // between the groups' phases were only keeping the two waves of a
        // SIMD in opposite roles (with them, eight per stage, 602 TOPS on the
        // sweep shape; without, 684 on the same box).  The copy of stage t+1
        // is stored with the first three groups' matrix work, one chunk each,
        // and group q's scale rows with group q's.  The buffer parity h is a
        // template constant here (the stage body is too large for the
        // compiler to unroll the loop below).
        auto stage32 = [&](auto hc, int t) __attribute__((always_inline)) {
            constexpr int h = decltype(hc)::value;
            if (EARLY) {
                load_stage(t + 2, h);
                mma_group(h, 0);
                store_stage(h ^ 1, h ^ 1, 0, 1, false);
                store_scales(h ^ 1, h ^ 1, 0, 1);
                rescale(4 * t);
                mma_group(h, 1);
                store_stage(h ^ 1, h ^ 1, 1, 2, false);
                store_scales(h ^ 1, h ^ 1, 1, 2);
                rescale(4 * t + 1);
                mma_group(h, 2);
                store_stage(h ^ 1, h ^ 1, 2, NCH, false);
                store_scales(h ^ 1, h ^ 1, 2, 3);
                rescale(4 * t + 2);
                mma_group(h, 3);
                store_scales(h ^ 1, h ^ 1, 3, 4);
                rescale(4 * t + 3);
                lds_barrier();
            } else {
                if (t > 0) rescale(4 * t - 1);
                load_stage(t + 2, h);
                mma_group(h, 0);
                store_stage(h ^ 1, h ^ 1, 0, 1, false);
                store_scales(h ^ 1, h ^ 1, 0, 1);
                rescale(4 * t);
                mma_group(h, 1);
                store_stage(h ^ 1, h ^ 1, 1, 2, false);
                store_scales(h ^ 1, h ^ 1, 1, 2);
                rescale(4 * t + 1);
                mma_group(h, 2);
                store_stage(h ^ 1, h ^ 1, 2, NCH, false);
                store_scales(h ^ 1, h ^ 1, 2, 3);
                rescale(4 * t + 2);
                mma_group(h, 3);
                store_scales(h ^ 1, h ^ 1, 3, 4);
                lds_barrier();
            }
        };
        for (int t0 = 0; t0 < stages; t0 += 2) {
            stage32(std::integral_constant<int, 0>{}, t0);
            if (t0 + 1 < stages) stage32(std::integral_constant<int, 1>{}, t0 + 1);
        }
    } else
    for (int t0 = 0; t0 < stages; t0 += 2)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int t = t0 + h;
        if (t >= stages) break;
        // (t and h have the same parity)
        const bool zero = SPG == 1 || (SPG == 2 && h == 0);   // stage t starts a group
        const bool ends = SPG == 1 || (SPG == 2 && h == 1);   // stage t ends a group
        const int grp = SPG == 2 ? t >> 1 : t;                // the group of stage t
        // The copy runs in every stage, also past the last one: loads past the
        // end of K read other rows or zeros, and the stores go to a buffer
        // that is no longer read; unconditional memory operations keep the
        // wait counts exact (the loads of stage t+2 stay in flight).
        if constexpr (F8) {
            // FP8 operands, groups of one stage: the ping-pong as below with
            // the copy's single register set stored (stage t+1) before the
            // loads of stage t+2 are issued into it.  Groups of 64: the same
            // per group, four phases per stage (the copy in the first matrix
            // phase).
            if constexpr (GN) {
                if (EARLY) {
                    store_stage(h ^ 1, 0);
                    load_stage(t + 2, 0);
                    mma_group(h, 0);
                    lds_barrier();
                    rescale(2 * t);
                    lds_barrier();
                    mma_group(h, 1);
                    lds_barrier();
                    rescale(2 * t + 1);
                    lds_barrier();
                } else {
                    if (t > 0) rescale(2 * t - 1);
                    lds_barrier();
                    store_stage(h ^ 1, 0);
                    load_stage(t + 2, 0);
                    mma_group(h, 0);
                    lds_barrier();
                    rescale(2 * t);
                    lds_barrier();
                    mma_group(h, 1);
                    lds_barrier();
                }
            } else if (EARLY) {
                store_stage(h ^ 1, 0);
                load_stage(t + 2, 0);
                mma_stage(h, true, true);
                lds_barrier();
                rescale(t);
                lds_barrier();
            } else {
                if (t > 0) rescale(t - 1);
                lds_barrier();
                store_stage(h ^ 1, 0);
                load_stage(t + 2, 0);
                mma_stage(h, true, true);
                lds_barrier();
            }
        } else if constexpr (GN) {
            // Groups of 64, ping-pong per group: four phases per stage, the
            // two groups' matrix work and rescales alternating as for groups
            // of one stage.  The copy of stage t+1 is stored in this stage's
            // matrix phases (its buffer was last read in the phase before
            // this stage's first): two chunks and the scale rows in the
            // first, one chunk in the second.  (Groups of 32 run the loop
            // below.)
            if constexpr (NG == 2) {
                if (EARLY) {
                    load_stage(t + 2, h);
                    mma_group(h, 0);
                    store_stage(h ^ 1, h ^ 1, 0, 2, true);
                    lds_barrier();
                    rescale(2 * t);
                    lds_barrier();
                    mma_group(h, 1);
                    store_stage(h ^ 1, h ^ 1, 2, NCH, false);
                    lds_barrier();
                    rescale(2 * t + 1);
                    lds_barrier();
                } else {
                    if (t > 0) rescale(2 * t - 1);
                    lds_barrier();
                    load_stage(t + 2, h);
                    mma_group(h, 0);
                    store_stage(h ^ 1, h ^ 1, 0, 2, true);
                    lds_barrier();
                    rescale(2 * t);
                    lds_barrier();
                    mma_group(h, 1);
                    store_stage(h ^ 1, h ^ 1, 2, NCH, false);
                    lds_barrier();
                }
            }
        } else {
        if (SPG == 0) {
            // One group over K: no per-stage rescale to overlap, so both wave
            // groups run the matrix work of every stage at the same time (two
            // waves per SIMD issuing MFMAs), one barrier per stage.
            load_stage(t + 2, h);
            mma_stage(h, zero, ends);
            store_stage(h ^ 1, h ^ 1);
            lds_barrier();
        } else if (SPG == 2) {
            // Groups of two stages: one rescale per two stages leaves the
            // ping-pong's vector phase empty half the time, so here too both
            // wave groups run the matrix work of every stage together, and
            // every wave rescales the group after the barrier of its second
            // stage.  The first stage stores its copy after the MFMAs (as for
            // one group over K); in the second, P is live from the first, so
            // the stored registers are freed before the MFMAs.
            load_stage(t + 2, h);
            if (h == 0) {
                mma_stage(h, zero, ends);
                store_stage(h ^ 1, h ^ 1);
            } else {
                store_stage(h ^ 1, h ^ 1);
                mma_stage(h, zero, ends);
            }
            lds_barrier();
            if (ends) rescale(grp);
        } else if (EARLY) {
            // groups of one stage, ping-pong.  Phase 1: matrix work of stage
            // t, most of the copy of stage t+1.  Phase 2: rescale of stage
            // t's group and the rest of the copy (the matrix phase is the
            // longer one: one of the thread's three chunks is stored here;
            // not in mixed mode, whose rescale is the longer).  Outside mixed
            // mode one barrier per stage: the copy goes to the buffer every
            // wave finished reading before the last barrier and is read after
            // the next, so the barrier between the phases only kept the two
            // waves of a SIMD in opposite roles (1524 -> 1567 TOPS on the
            // sweep shape and +2.6% on the 70B prefill layers, one box)
            load_stage(t + 2, h);
            mma_stage(h, true, true);
            store_stage(h ^ 1, h ^ 1, 0, SPLIT, true);
            if (MIXED) lds_barrier();
            rescale(t);
            store_stage(h ^ 1, h ^ 1, SPLIT, NCH, false);
            lds_barrier();
        } else {
            // phase 1: rescale of stage t-1's group, the vector phase's part
            // of the copy of stage t+1 (its buffer was last read in stage
            // t-1); phase 2: matrix work of stage t, the rest of the copy
            if (t > 0) rescale(t - 1);
            store_stage(h ^ 1, h ^ 1, SPLIT, NCH, false);
            if (MIXED) lds_barrier();
            load_stage(t + 2, h);
            mma_stage(h, true, true);
            store_stage(h ^ 1, h ^ 1, 0, SPLIT, true);
            lds_barrier();
        }
        }
    }
    if (SPG == 0) {
        // one group: its scale products from the last stage's buffer (the
        // scales are the same in every stage)
        scale_products((stages - 1) & 1);
        rescale(0);
    } else if (!EARLY && SPG == 1) {
        // the last stage ends the last group
        rescale(stages - 1);
    } else if (!EARLY && GN) {
        rescale(NG * stages - 1);
    }

    if (a.part) {
        // K-split part: the tile's fp32 sums, all BM x BN of them
        float* out = a.part + (size_t)(kpart * a.ntail + lin) * (BM * BN);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    out[(wm * 64 + mt * 32 + acc_row(r, lane)) * BN + wn * 64 + nt * 32 + (lane & 31)] =
                        acc[mt][nt][r];
        return;
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
                    // keep the fp32 value: the multiply and the fp16 conversion
                    // must not fuse into one rounding (y16 is the fp16 of y32)
                    asm volatile("" : "+v"(v));
                    const int64_t o = (int64_t)m * a.N + n;
                    a.y16[o] = (_Float16)v;
                    if (a.y32) a.y32[o] = v;
                }
            }
        }
}

template <bool MIXED, bool DEBUG_P, int SPG, bool F8 = false>
__global__ __launch_bounds__(THREADS, 2) void gemm_pp_kernel(PPArgs a)
{
    __shared__ PPShared<PPMode<SPG>::NG, PPMode<SPG>::HV> sh;
    // wave-uniform role (a scalar branch)
    if (__builtin_amdgcn_readfirstlane(threadIdx.x) < THREADS / 2)
        pp_body<MIXED, DEBUG_P, SPG, true, F8>(a, sh);
    else
        pp_body<MIXED, DEBUG_P, SPG, false, F8>(a, sh);
}

// Y of the K-split tiles: the parts' sums added in part order, then as the
// epilogue above (mixed: x s_w[n]; fp16 is the RNE rounding of the fp32
// value).  One thread per 4 consecutive columns of a tile row.
template <bool MIXED>
__global__ __launch_bounds__(256) void pp_split_reduce_kernel(PPArgs a)
{
    const int idx = blockIdx.x * 256 + threadIdx.x;
    constexpr int PER_TILE = BM * BN / 4;
    if (idx >= a.ntail * PER_TILE) return;
    const int lin = idx / PER_TILE, rem = idx - lin * PER_TILE;
    const int row = rem / (BN / 4), col = (rem - row * (BN / 4)) * 4;
    const int tile = a.tile0 + lin;
    int by, bx;
    tile_coords(a, tile, by, bx);
    const int m = by * BM + row;
    if (m >= a.M) return;
    const size_t o0 = (size_t)lin * (BM * BN) + row * BN + col;
    const size_t stride = (size_t)a.ntail * (BM * BN);
    const float4 p0 = *reinterpret_cast<const float4*>(a.part + o0);
    float s[4] = {p0.x, p0.y, p0.z, p0.w};
    for (int q = 1; q < a.nparts; ++q) {
        const float4 pq = *reinterpret_cast<const float4*>(a.part + q * stride + o0);
        s[0] += pq.x;
        s[1] += pq.y;
        s[2] += pq.z;
        s[3] += pq.w;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int n = bx * BN + col + j;
        if (n < a.N) {
            float v = MIXED ? s[j] * a.sw[n] : s[j];
            asm volatile("" : "+v"(v));
            const int64_t o = (int64_t)m * a.N + n;
            a.y16[o] = (_Float16)v;
            if (a.y32) a.y32[o] = v;
        }
    }
}

template <bool MIXED, int SPG>
void launch_pp(const PPArgs& t, int grid, hipStream_t stream)
{
    if (t.psum) gemm_pp_kernel<MIXED, true, SPG><<<grid, THREADS, 0, stream>>>(t);
    else gemm_pp_kernel<MIXED, false, SPG><<<grid, THREADS, 0, stream>>>(t);
}

template <bool MIXED, int SPG>
void launch_pp_all(const PPArgs& t, const PingpongSplit& sp, hipStream_t stream)
{
    if (sp.tail == 0) {
        launch_pp<MIXED, SPG>(t, sp.tiles, stream);
        return;
    }
    // the full rounds of tiles over all of K, then the last (partial) round
    // as nparts K parts on nparts times the workgroups, then their sums
    if (sp.tiles > sp.tail) launch_pp<MIXED, SPG>(t, sp.tiles - sp.tail, stream);
    PPArgs k = t;
    k.tile0 = sp.tiles - sp.tail;
    k.ntail = sp.tail;
    k.nparts = sp.nparts;
    k.part = sp.part;
    launch_pp<MIXED, SPG>(k, sp.nparts * sp.tail, stream);
    pp_split_reduce_kernel<MIXED><<<(sp.tail * (BM * BN / 4) + 255) / 256, 256, 0, stream>>>(k);
}

// Row blocks per band of the tile order: 16 (a round of 256 workgroups then
// covers 16 x 16 tiles: at K = 8192 their A and B blocks are 24 MB, against
// 129 MB for one row block and 256 column blocks in row-major order).
// row blocks per band: 32 consecutive tiles (one XCD's workgroups in flight)
// cover 4 row blocks x 8 column blocks
int tile_band_rows(int tiles_m) { return tiles_m < 4 ? tiles_m : 4; }

int cu_count()
{
    // compute units of the current device, cached per device (relaxed atomics:
    // concurrent first calls store the same value)
    static std::atomic<int> cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

}  // namespace

PingpongSplit pingpong_split(const GemmProblem& p)
{
    // One workgroup per CU (the LDS of one fills a CU), so a launch runs in
    // rounds of `cus` tiles.  When the last round (the only one, for few
    // tiles) is at most half full, its tiles are split over K into
    // nparts = min(cus / tiles, stages / 2, 4) parts (at group boundaries:
    // groups of one stage or half a stage only), which fills up to nparts times as many CUs
    // for 1/nparts of the time; the reduction reads nparts partial tiles
    // (more parts measured slower: their fp32 partial tiles cost more traffic
    // than the shorter K saves).
    PingpongSplit sp;
    sp.tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
    const int gs = p.ga < p.gw ? p.ga : p.gw;
    const int cus = cu_count();
    const int stages = p.K / KSTAGE;
    if ((gs != KSTAGE && gs != KSTAGE / 2 && gs != KSTAGE / 4) || stages < 4 || cus <= 0) return sp;
    const int tail = sp.tiles % cus;
    if (tail == 0 || 2 * tail > cus) return sp;
    int parts = cus / tail;
    if (parts > stages / 2) parts = stages / 2;
    if (parts > 4) parts = 4;
    sp.tail = tail;
    sp.nparts = parts;
    sp.bytes = (size_t)parts * tail * BM * BN * sizeof(float);
    return sp;
}

bool pingpong_supports(const GemmProblem& p)
{
    const int gs = p.ga < p.gw ? p.ga : p.gw;
    const bool mixed = p.gw == p.K && p.ga != p.gw;
    // groups of a quarter stage (32), half a stage (64), one stage (128), two
    // stages (256) or one group (K); mixed mode with activation groups of
    // half a stage, one or two stages
    if (!(gs == KSTAGE / 4 || gs == KSTAGE / 2 || gs == KSTAGE || gs == 2 * KSTAGE ||
          (gs == p.K && gs % KSTAGE == 0)))
        return false;
    if (p.K % KSTAGE != 0) return false;
    if (!mixed && p.ga != p.gw) return false;
    if (mixed && p.ga != KSTAGE / 2 && p.ga != KSTAGE && p.ga != 2 * KSTAGE) return false;
    // 32-bit buffer offsets within one workgroup's rows
    const uint64_t rowbytes = (uint64_t)p.K / 2;
    return rowbytes * BM < (1ull << 31) && (uint64_t)p.K / gs * 4 * BM < (1ull << 31);
}

hipError_t launch_gemm_pingpong_f8(const GemmProblem& p, hipStream_t stream)
{
    // FP8-coded operands (qa, qw: [rows, K] bytes), groups of 128 (one stage
    // per group) or 64 (two per stage) on both operands
    PPArgs t{};
    t.qa = p.qa;
    t.sa = p.sa;
    t.qw = p.qw;
    t.sw = p.sw;
    t.M = p.M;
    t.N = p.N;
    t.K = p.K;
    const int g = p.ga;   // 64 or 128, both operands
    t.Ga = p.K / g;
    t.Gw = p.K / g;
    t.spg = g == KSTAGE / 2 ? -1 : 1;
    t.G = p.K / g;
    t.y16 = static_cast<_Float16*>(p.y16);
    t.y32 = p.y32;
    t.psum = p.psum;
    t.prows = p.prows;
    t.tiles_n = (p.N + BN - 1) / BN;
    t.tiles_m = (p.M + BM - 1) / BM;
    t.group_m = tile_band_rows(t.tiles_m);
    t.nparts = 1;
    const int tiles = ((p.M + BM - 1) / BM) * t.tiles_n;
    if (g == KSTAGE / 2) {
        if (t.psum) gemm_pp_kernel<false, true, -1, true><<<tiles, THREADS, 0, stream>>>(t);
        else gemm_pp_kernel<false, false, -1, true><<<tiles, THREADS, 0, stream>>>(t);
    } else {
        if (t.psum) gemm_pp_kernel<false, true, 1, true><<<tiles, THREADS, 0, stream>>>(t);
        else gemm_pp_kernel<false, false, 1, true><<<tiles, THREADS, 0, stream>>>(t);
    }
    return hipGetLastError();
}

hipError_t launch_gemm_pingpong(const GemmProblem& p, hipStream_t stream)
{
    PPArgs t;
    t.qa = p.qa;
    t.sa = p.sa;
    t.qw = p.qw;
    t.sw = p.sw;
    t.M = p.M;
    t.N = p.N;
    t.K = p.K;
    t.Ga = p.K / p.ga;
    t.Gw = p.K / p.gw;
    const int gs = p.ga < p.gw ? p.ga : p.gw;
    t.spg = gs == KSTAGE / 2 ? -1 : gs == KSTAGE / 4 ? -2 : gs / KSTAGE;
    t.G = p.K / gs;
    t.y16 = static_cast<_Float16*>(p.y16);
    t.y32 = p.y32;
    t.psum = p.psum;
    t.prows = p.prows;
    t.tiles_n = (p.N + BN - 1) / BN;
    t.tiles_m = (p.M + BM - 1) / BM;
    t.group_m = tile_band_rows(t.tiles_m);
    t.tile0 = 0;
    t.ntail = 0;
    t.nparts = 1;
    t.part = nullptr;
    PingpongSplit sp = pingpong_split(p);
    // the K split needs its workspace (each part writes the debug sums of
    // its own groups)
    if (sp.tail && (!p.ws || p.ws_bytes < sp.bytes)) sp.tail = 0;
    sp.part = static_cast<float*>(p.ws);
    const bool mixed = p.gw == p.K && p.ga != p.gw;
    // mixed mode here: ga = 64, 128 or 256 (the activation groups are half a
    // stage, 1 or 2 stages)
    if (mixed && gs == KSTAGE / 2) launch_pp_all<true, -1>(t, sp, stream);
    else if (mixed && t.spg == 1) launch_pp_all<true, 1>(t, sp, stream);
    else if (mixed) launch_pp_all<true, 2>(t, sp, stream);
    else if (gs == KSTAGE / 2) launch_pp_all<false, -1>(t, sp, stream);
    else if (gs == KSTAGE / 4) launch_pp_all<false, -2>(t, sp, stream);
    else if (t.spg == 1) launch_pp_all<false, 1>(t, sp, stream);
    else if (gs == p.K) launch_pp_all<false, 0>(t, sp, stream);
    else launch_pp_all<false, 2>(t, sp, stream);
    return hipGetLastError();
}

}  // namespace apex4
