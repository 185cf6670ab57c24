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
// Work split.  A workgroup of 4, 8 or 16 waves owns 32 output columns and all M
// rows (16x16 MFMA tiles: ceil(M/16) row tiles, 2 column tiles).  The waves
// split K among themselves in runs of consecutive 128-value chunks (two
// groups at g = 128, else whole groups), run q going to wave q mod W, so each
// wave reads whole 128-byte lines of 32 weight rows with 16-byte loads while
// the other waves stream the neighbouring lines.  Each wave keeps the loads of
// the next few chunks, and the scales of the groups they complete, in flight.
// At the end the partial fp32 tiles are summed through LDS in a fixed order.
// When the whole row is one group (per-channel scales on both operands) the
// waves instead add their int32 partial sums exactly before the single
// rescale.
//
// K order inside a chunk: lane block kb (lanes 16kb..16kb+15) holds the 32
// codes of bytes [16kb, 16kb+16); the first 16 feed K-step 0 and the last 16
// K-step 1.  The same assignment is used for both operands, so each MFMA sums
// the products of one chunk, i.e. of one group (groups are >= 128 here).
#include "internal.h"

namespace apex4 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int BN = 32;                         // output columns per workgroup
constexpr int CHUNK = 128;                     // K values per chunk (64 packed bytes per row)

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
    PsumRows prows;
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

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Offsets at or past this are outside every buffer below: the hardware range
// check of a raw buffer load returns 0 for them, which is how rows past M or
// N and chunks past K are read without any branch.
constexpr uint32_t OOB = 0x80000000u;

__device__ inline __amdgpu_buffer_rsrc_t buffer_of(const void* p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

__device__ inline uint4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ inline float load_f32(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}

// LDS layout of one workgroup (dynamic shared memory, sizes in floats):
//   scale_a [Ga][16*MT]  activation scales, group-major (x 2^-8)
//   scale_w [Gw][32]     weight scales of the 32 columns, group-major
//   red     [W][MT][2][4][64]  cross-wave reduction
struct SkinnyLds {
    int sa_off, sw_off, red_off, bytes;
};

__host__ __device__ inline SkinnyLds skinny_lds(int MT, int W, int Ga, int Gw, bool one_group)
{
    SkinnyLds l;
    const int na = one_group ? 0 : Ga * 16 * MT;
    const int nw = one_group ? 0 : Gw * BN;
    l.sa_off = 0;
    l.sw_off = na;
    l.red_off = na + nw;
    l.bytes = 4 * (na + nw + W * MT * 2 * 4 * 64);
    return l;
}

// MT: 16-row tiles (ceil(M/16)).  W: waves per workgroup.  Up to 48 rows the
// kernel keeps to 128 VGPRs (4 waves per SIMD, 16 per CU); 64 rows need the
// registers of 2 waves per SIMD.  Each wave has 4 chunks of loads in flight
// at 16 rows, 3 at 32 and 2 above.  ONE_GROUP: gs == K, the waves split
// the chunks of the single group and add their int32 sums before rescaling.
//
// The scales a workgroup needs are copied to LDS once, before the chunk loop,
// so the loop issues only the three operand loads per chunk.  The loop has no
// branch around a load: the loads of a chunk are always issued (out-of-range
// ones read zeros), so the compiler can leave the loads of the following
// chunks in flight while one chunk is multiplied.
template <int MT, int W, bool MIXED, bool DEBUG_P, bool ONE_GROUP>
__global__ __launch_bounds__(W * 64, MT <= 3 ? 4 : 2) void gemm_skinny_kernel(SkinnyArgs a)
{
    constexpr int PREFETCH = MT == 1 ? 4 : (MT == 2 ? 3 : 2);
    extern __shared__ __attribute__((aligned(16))) float lds[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wave-uniform by construction; saying so lets the chunk bookkeeping below
    // live in scalar registers instead of per-lane branches
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 15, kb = lane >> 4;
    const int n0 = blockIdx.x * BN;
    const uint32_t rowbytes = (uint32_t)a.K / 2;
    const int cpg = a.gs / CHUNK;             // chunks per group
    const int total_chunks = a.K / CHUNK;
    const SkinnyLds L = skinny_lds(MT, W, a.Ga, MIXED ? 0 : a.Gw, ONE_GROUP);
    float* lsa = lds + L.sa_off;
    float* lsw = lds + L.sw_off;
    float* red = lds + L.red_off;

    if (!ONE_GROUP) {
        // scales -> LDS, group-major; rows past M / columns past N get 0
        const int rows = 16 * MT;
        for (int idx = tid; idx < rows * a.Ga; idx += W * 64) {
            const int m = idx / a.Ga, j = idx - m * a.Ga;
            lsa[j * rows + m] = m < a.M ? a.sa[(int64_t)m * a.Ga + j] * 0.00390625f : 0.0f;
        }
        if (!MIXED) {
            for (int idx = tid; idx < BN * a.Gw; idx += W * 64) {
                const int c = idx / a.Gw, j = idx - c * a.Gw;
                lsw[j * BN + c] = n0 + c < a.N ? a.sw[(int64_t)(n0 + c) * a.Gw + j] : 0.0f;
            }
        }
        __syncthreads();
    }

    const __amdgpu_buffer_rsrc_t ra = buffer_of(a.qa, (uint32_t)a.M * rowbytes);
    const __amdgpu_buffer_rsrc_t rb = buffer_of(a.qw, (uint32_t)a.N * rowbytes);

    // byte offset of this lane's operand row (OOB past M / N)
    uint32_t offa[MT], offb[2];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int m = 16 * mt + li;
        offa[mt] = m < a.M ? (uint32_t)m * rowbytes + 16 * kb : OOB;
    }
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const int n = n0 + 16 * nt + li;
        offb[nt] = n < a.N ? (uint32_t)n * rowbytes + 16 * kb : OOB;
    }

    // This wave's chunks come in runs of consecutive chunks, so that each
    // wave reads whole 128-byte lines of every weight row: runs of 2 chunks
    // (two groups) when gs = 128 or the row is one group, else whole groups;
    // run q of this wave is run number wave + W*q.  Every wave walks the same
    // number of items; items past K are out-of-range reads of zeros.
    const int run = (cpg == 1 || ONE_GROUP) ? 2 : cpg;
    const int runs = (total_chunks + run - 1) / run;
    const int n_items = ((runs + W - 1) / W) * run;
    auto chunk_of = [&](int i) -> int {
        const int q = i / run;
        return (wave + W * q) * run + (i - q * run);
    };

    uint4 bufA[PREFETCH][MT], bufB[PREFETCH][2];
    auto issue = [&](int slot, int i) {
        // Offsets: a row past M / N starts at OOB and a chunk adds less than
        // 2^30, so the sum stays in [OOB, 2^32); a chunk past K is OOB itself.
        const int c = chunk_of(i);
        const bool live = c < total_chunks;
        const uint32_t koff = (uint32_t)c * (CHUNK / 2);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) bufA[slot][mt] = load16(ra, live ? offa[mt] + koff : OOB);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) bufB[slot][nt] = load16(rb, live ? offb[nt] + koff : OOB);
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

    for (int i0 = 0; i0 < n_items; i0 += PREFETCH) {
#pragma unroll
        for (int k = 0; k < PREFETCH; ++k) {
            const int i = i0 + k;
            issue((k + PREFETCH - 1) % PREFETCH, i + PREFETCH - 1);
            const int c = chunk_of(i);
            const bool first = ONE_GROUP ? (i == 0) : (c % cpg == 0);
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
                    v4i cc = first ? v4i{} : P[mt][nt];
                    cc = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[mt][0], fb[nt][0], cc, 0, 0, 0);
                    P[mt][nt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[mt][1], fb[nt][1], cc, 0, 0, 0);
                }
            if (!ONE_GROUP && (c + 1) % cpg == 0 && c < total_chunks) {
                // the group is complete: rescale into acc
                const int j = c / cpg;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const float4 sa4 = *reinterpret_cast<const float4*>(&lsa[j * 16 * MT + 16 * mt + 4 * kb]);
                    const float sa[4] = {sa4.x, sa4.y, sa4.z, sa4.w};
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) {
                        const float sw = MIXED ? 1.0f : lsw[j * BN + 16 * nt + li];
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const float S = MIXED ? sa[r] : sa[r] * sw;
                            acc[mt][nt][r] = fmaf(S, (float)P[mt][nt][r], acc[mt][nt][r]);
                        }
                    }
                }
                if (DEBUG_P) {
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                        for (int nt = 0; nt < 2; ++nt) {
                            const int n = n0 + 16 * nt + li;
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                const int m = 16 * mt + 4 * kb + r;
                                if (m < a.M && n < a.N)
                                    if (int32_t* d = psum_at(a.psum, a.prows, m, n, a.N, a.G, j))
                                        *d = P[mt][nt][r] >> 8;
                            }
                        }
                }
            }
        }
    }

    if (ONE_GROUP) {
        // exact int32 sum of the waves' partial sums, then one rescale
        int* redi = reinterpret_cast<int*>(red);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    redi[(((wave * MT + mt) * 2 + nt) * 4 + r) * 64 + lane] = P[mt][nt][r];
        __syncthreads();
        for (int o = tid; o < MT * 2 * 4 * 64; o += W * 64) {
            const int ln = o & 63, r = (o >> 6) & 3, nt = (o >> 8) & 1, mt = o >> 9;
            const int m = 16 * mt + 4 * (ln >> 4) + r;
            const int n = n0 + 16 * nt + (ln & 15);
            if (m < a.M && n < a.N) {
                int p = 0;
                for (int w = 0; w < W; ++w) p += redi[(((w * MT + mt) * 2 + nt) * 4 + r) * 64 + ln];
                const float S = a.sa[m] * 0.00390625f * a.sw[n];
                float v = S * (float)p;
                asm volatile("" : "+v"(v));
                const int64_t off = (int64_t)m * a.N + n;
                a.y16[off] = (_Float16)v;
                if (a.y32) a.y32[off] = v;
                if (DEBUG_P)
                    if (int32_t* d = psum_at(a.psum, a.prows, m, n, a.N, 1, 0)) *d = p >> 8;
            }
        }
        return;
    }

    // sum the partial tiles of the waves in a fixed order, then write
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[(((wave * MT + mt) * 2 + nt) * 4 + r) * 64 + lane] = acc[mt][nt][r];
    __syncthreads();
    for (int o = tid; o < MT * 2 * 4 * 64; o += W * 64) {
        const int ln = o & 63, r = (o >> 6) & 3, nt = (o >> 8) & 1, mt = o >> 9;
        const int m = 16 * mt + 4 * (ln >> 4) + r;
        const int n = n0 + 16 * nt + (ln & 15);
        if (m < a.M && n < a.N) {
            float v = 0.0f;
            for (int w = 0; w < W; ++w) v += red[(((w * MT + mt) * 2 + nt) * 4 + r) * 64 + ln];
            if (MIXED) v *= a.sw[n];
            asm volatile("" : "+v"(v));
            const int64_t off = (int64_t)m * a.N + n;
            a.y16[off] = (_Float16)v;
            if (a.y32) a.y32[off] = v;
        }
    }
}

template <int MT, int W>
void launch_mt(const SkinnyArgs& s, bool mixed, bool dbg, bool one, hipStream_t stream)
{
    dim3 grid((s.N + BN - 1) / BN);
    const size_t lds = skinny_lds(MT, W, s.Ga, mixed ? 0 : s.Gw, one).bytes;
#define APEX4_SKINNY(MX, DB, ONE) gemm_skinny_kernel<MT, W, MX, DB, ONE><<<grid, W * 64, lds, stream>>>(s)
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

// Waves per workgroup: about one round of 16 waves on each of the 256 CUs
// (N/32 column blocks x W waves ~ 4096), so the K split is as wide as the
// column count allows and no workgroups are left for a second round; capped
// by what the workgroup's LDS tables allow.
int skinny_waves(int mt, int N, int Ga, int Gw, bool one)
{
    const int blocks = (N + BN - 1) / BN;
    const int max_lds = 160 * 1024;
    const int cand[3] = {16, 8, 4};
    for (int w : cand) {
        if (w == 16 && (mt > 3 || blocks > 256)) continue;
        if (w == 8 && blocks > (mt <= 3 ? 512 : 256)) continue;
        if (skinny_lds(mt, w, Ga, Gw, one).bytes <= max_lds) return w;
    }
    return skinny_lds(mt, 4, Ga, Gw, one).bytes <= max_lds ? 4 : 0;
}

template <int MT>
void launch_waves(const SkinnyArgs& s, bool mixed, bool dbg, bool one, hipStream_t stream)
{
    const int w = skinny_waves(MT, s.N, s.Ga, mixed ? 0 : s.Gw, one);
    if constexpr (MT <= 3) {
        if (w == 16) {
            launch_mt<MT, 16>(s, mixed, dbg, one, stream);
            return;
        }
    }
    if (w == 8)
        launch_mt<MT, 8>(s, mixed, dbg, one, stream);
    else
        launch_mt<MT, 4>(s, mixed, dbg, one, stream);
}

}  // namespace

bool skinny_supports(const GemmProblem& p)
{
    // buffer offsets are 32-bit and must stay below the OOB marker
    const int gs = p.ga < p.gw ? p.ga : p.gw;
    const uint64_t wbytes = (uint64_t)p.N * (p.K / 2), abytes = (uint64_t)p.M * (p.K / 2);
    const uint64_t swbytes = (uint64_t)p.N * (p.K / p.gw) * 4;
    const uint64_t sabytes = (uint64_t)p.M * (p.K / p.ga) * 4;
    // the per-workgroup scale tables must fit in LDS next to the reduction buffer
    const bool one = gs == p.K;
    const bool mixed = (p.gw == p.K) && (p.ga != p.gw);
    const int mt = (p.M + 15) / 16;
    if (p.M < 1 || p.M > 64) return false;
    const int w = skinny_waves(mt, p.N, p.K / p.ga, mixed ? 0 : p.K / p.gw, one);
    return gs >= CHUNK && wbytes < OOB && abytes < OOB && swbytes < OOB && sabytes < OOB &&
           p.K < (1 << 30) && w > 0;
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
    s.prows = p.prows;
    const bool mixed = (p.gw == p.K) && (p.ga != p.gw);
    const bool one = s.gs == p.K;
    const bool dbg = p.psum != nullptr;
    const int mt = (p.M + 15) / 16;
    switch (mt) {
    case 1: launch_waves<1>(s, mixed, dbg, one, stream); break;
    case 2: launch_waves<2>(s, mixed, dbg, one, stream); break;
    case 3: launch_waves<3>(s, mixed, dbg, one, stream); break;
    default: launch_waves<4>(s, mixed, dbg, one, stream); break;
    }
    return hipGetLastError();
}

}  // namespace apex4
