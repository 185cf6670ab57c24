// W4A4 GEMM with per-group dequantization on FP6-coded operands (gfx950),
// groups of 128 on both operands, for compute-bound calls.
//
// The computation is the APEX4 page's (Abstract): INT4 x INT4 products summed
// exactly per K-group, every group's sum rescaled by s_a*s_w and accumulated
// in fp32.  The OSC page (Abstract) points to 4-bit micro-scaling matrix
// hardware for this kind of arithmetic.  gfx950's micro-scaling instruction
// v_mfma_scale_f32_32x32x64_f8f6f4 takes FP6 operands at twice the int8
// matrix rate and sums their products in fp32.  The INT4 codes travel in the
// FP6 E2M3 format: the field (c < 0) << 5 | |c| is the value c / 8 exactly
// (apex4_quantize_f6), the instruction's E8M0 block scales multiply both
// operands back by 2^3, and the fp32 sum of 64 products of integers of at
// most 8 in magnitude is exact, so every group sum P equals the integer one.
//
// Against the nibble kernels this removes, per stage and wave, the widening
// of the codes (they are MFMA operands as stored), the copy's trip through
// VGPRs and LDS stores (the packed rows go straight from memory to LDS with
// buffer_load ... lds), and the int32 -> fp32 conversion of the rescale (one
// fma per output and group).  The price is 6 bits of storage per code.
//
// Workgroup: 8 waves on a 256x128 tile of Y, each wave 64x64 = four 32x32
// tiles; K advances in stages of 128 (one group).  LDS holds three stage
// buffers, filled two stages ahead.  A stage buffer stores the 96 bytes of a
// row's stage as six 16-byte chunk planes (plane q holds chunk q of every
// row): the operands' tiled layout (apex4_quantize_f6) has chunk q of 64
// rows and one group as a contiguous KB, so one direct-to-LDS load of whole
// 64-lane pieces fills it, and the fragment reads of 16 consecutive rows are
// conflict-free.  (A row-major operand would need 64 scattered 16-byte
// pieces per load; that copy ran at half the speed.)  K order inside a
// group: lanes 0..31 of a 32x64 MFMA operand hold codes 0..31 (K-step 0) and
// 32..63 (step 1) of their row, lanes 32..63 codes 64..95 and 96..127: the
// same permutation on both operands, so the group sum is unchanged, and each
// lane's 48 bytes are three whole chunks.
//
// In window i of a stage a wave issues the two FP6 MFMAs of tile T_i with
// the bf16 MFMA of its scale product S_i between them (exact three-piece
// bf16 splits of s_a and s_w, six of the nine cross products, as in the
// nibble kernels), then the 16 fmas that fold the previous tile's group sum
// into its accumulators: that sum was finished three matrix instructions
// earlier, so the fold does not wait on it (folding it between this tile's
// MFMAs, right after its last K-step was issued, stalled there).
#include "internal.h"

namespace apex4 {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int BM = 256;
constexpr int BN = 128;
constexpr int THREADS = 512;
constexpr int HALF = THREADS / 2;
constexpr int KSTAGE = 128;             // K values per stage (one group)
constexpr int ROWB = KSTAGE * 3 / 4;    // FP6 bytes per row per stage
constexpr int PLANES = ROWB / 16;       // 16-byte chunk planes per stage
constexpr int TILE_BYTES = PLANES * 64 * 16;   // one (64-row block, group) tile of the operands
// direct-to-LDS loads per stage: one per (plane, 64 rows)
constexpr int LOADS_A = PLANES * BM / 64;
constexpr int LOADS = LOADS_A + PLANES * BN / 64;
// E8M0 block scale 2^3 (biased exponent 127 + 3): the codes are stored as c / 8
constexpr int SCALE_E8M0 = 130;
constexpr int FMT_FP6 = 2;              // E2M3 operand format of the f8f6f4 instruction

struct F6Args {
    const uint8_t* qa;
    const float* sa;
    const uint8_t* qw;
    const float* sw;
    int M, N, K;
    int G;             // groups (K / 128): scale columns of both operands
    _Float16* y16;
    float* y32;
    int32_t* psum;
    PsumRows prows;
    int tiles_m, tiles_n;
    int group_m;       // row blocks walked per column block (tile order)
    int tile0;
    int ntail;
    int nparts;
    float* part;
};

// One stage buffer: chunk planes of A and B, and the scale operand rows
// (16 bytes per tile row: the eight K slots of the split-operand MFMA).
struct StageBuf {
    uint4 a[PLANES][BM];
    uint4 b[PLANES][BN];
    uint2 ta[2][BM];
    uint2 tb[2][BN];
};

__device__ inline __amdgpu_buffer_rsrc_t buffer_of(const void* p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

__device__ inline uint32_t bf16_trunc_bits(float x) { return __builtin_bit_cast(uint32_t, x) >> 16; }

__device__ inline void split3(float s, uint32_t& x0, uint32_t& x1, uint32_t& x2)
{
    x0 = bf16_trunc_bits(s);
    const float r1 = s - __builtin_bit_cast(float, x0 << 16);
    x1 = bf16_trunc_bits(r1);
    const float r2 = r1 - __builtin_bit_cast(float, x1 << 16);
    x2 = bf16_trunc_bits(r2);
}

__device__ inline int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// Workgroup barrier after this wave's LDS stores have completed.  (Not a
// release fence: on LDS that would also wait for every direct-to-LDS load in
// flight, i.e. drain the copy of the stage after next.  The copies a barrier
// must cover are waited for explicitly before it.)  The memory clobber keeps
// the compiler from moving memory accesses across it.
__device__ inline void lds_barrier()
{
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

__device__ inline void fence_sched() { __builtin_amdgcn_sched_barrier(0); }

__device__ inline void anchor4(float& a, float& b, float& c, float& d)
{
    asm volatile("" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
}
__device__ inline void anchor16(v16f& x) { asm volatile("" : "+v"(x)); }

__device__ inline void tile_coords(const F6Args& a, int tile, int& by, int& bx)
{
    const int band = a.group_m * a.tiles_n;
    const int g = tile / band;
    const int first = g * a.group_m;
    const int rows = min(a.group_m, a.tiles_m - first);
    const int local = tile - g * band;
    by = first + local % rows;
    bx = local / rows;
}

// the K-step s operand (32 codes, six dwords) out of a lane's three chunks
__device__ inline v8i step_operand(const uint4 (&c)[3], int s)
{
    if (s == 0) return v8i{(int)c[0].x, (int)c[0].y, (int)c[0].z, (int)c[0].w, (int)c[1].x, (int)c[1].y, 0, 0};
    return v8i{(int)c[1].z, (int)c[1].w, (int)c[2].x, (int)c[2].y, (int)c[2].z, (int)c[2].w, 0, 0};
}

// EARLY: waves 0..3 (the A scales); otherwise waves 4..7 (the B scales)
template <bool DEBUG_P, bool EARLY>
__device__ __forceinline__ void f6_body(const F6Args& a, StageBuf& b0, StageBuf& b1, StageBuf& b2)
{
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    int lin = blockIdx.x, kpart = 0;
    if (a.part) {
        kpart = lin / a.ntail;
        lin -= kpart * a.ntail;
    } else {
        // XCD-aware order, as in the nibble ping-pong kernel: the chip deals
        // workgroup b to XCD b mod 8 (each with its own L2), which then walks
        // a contiguous range of tile ids (bands of 4 row blocks)
        const int per = (int)gridDim.x >> 3;
        if (lin < per * 8) lin = (lin & 7) * per + (lin >> 3);
    }
    int by, bx;
    tile_coords(a, a.tile0 + lin, by, bx);
    const int m0 = by * BM, n0 = bx * BN;
    const int all_stages = a.K / KSTAGE;
    const int s0 = a.part ? kpart * all_stages / a.nparts : 0;
    const int stages = a.part ? (kpart + 1) * all_stages / a.nparts - s0 : all_stages;
    const int rows_a = min(BM, a.M - m0), rows_b = min(BN, a.N - n0);
    // the tiles of this workgroup's row blocks (6 KB per 64 rows and group);
    // blocks past the last one lie past the end of the buffer and read zeros
    const uint32_t block_bytes = (uint32_t)a.G * TILE_BYTES;
    const __amdgpu_buffer_rsrc_t rA = buffer_of(a.qa + (int64_t)(m0 / 64) * block_bytes,
                                                (uint32_t)((rows_a + 63) / 64) * block_bytes);
    const __amdgpu_buffer_rsrc_t rB = buffer_of(a.qw + (int64_t)(n0 / 64) * block_bytes,
                                                (uint32_t)((rows_b + 63) / 64) * block_bytes);
    const __amdgpu_buffer_rsrc_t rSA = buffer_of(a.sa + (int64_t)m0 * a.G, (uint32_t)rows_a * a.G * 4);
    const __amdgpu_buffer_rsrc_t rSW = buffer_of(a.sw + (int64_t)n0 * a.G, (uint32_t)rows_b * a.G * 4);

    // --- the direct-to-LDS copy of stage t into stage buffer d: this wave's
    // loads u = wave, wave + 8, ... of the LOADS (plane, 64-row block) pieces,
    // each a contiguous KB of the tiled operand (chunk q of the block's 64
    // rows; lane l brings row l's) ---
    constexpr int MY_LOADS = EARLY ? (LOADS + 7 - 0) / 8 : LOADS / 8;   // waves 0..3: 5, 4..7: 4
    auto copy_stage = [&](StageBuf& d, int t) {
#pragma unroll
        for (int j = 0; j < MY_LOADS; ++j) {
            const int u = wave + 8 * j;
            const bool is_a = u < LOADS_A;
            const int v = is_a ? u : u - LOADS_A;
            const int q = v / (is_a ? BM / 64 : BN / 64), blk = v % (is_a ? BM / 64 : BN / 64);
            const int off = (int)((((uint32_t)blk * a.G + (uint32_t)(s0 + t)) * PLANES + q) * 1024 + 16 * lane);
            lds_void* dst = is_a ? (lds_void*)&d.a[q][64 * blk] : (lds_void*)&d.b[q][64 * blk];
            __builtin_amdgcn_raw_ptr_buffer_load_lds(is_a ? rA : rB, dst, 16, off, 0, 0, 0);
        }
    };
    // scales: thread ht of waves 0..3 owns A row ht, of waves 4..7 B row ht
    // (threads past row 127 load from past the end: zeros, unused)
    const int ht = EARLY ? tid : tid - HALF;
    const bool has_scale = EARLY || ht < BN;
    const uint32_t soff = !has_scale ? 0x80000000u : (uint32_t)ht * a.G * 4;
    auto load_scale = [&](int t) {
        return __builtin_bit_cast(float,
                                  __builtin_amdgcn_raw_buffer_load_b32(EARLY ? rSA : rSW, (int)soff, (s0 + t) * 4, 0));
    };
    auto store_scale = [&](StageBuf& d, float sc) {
        if (EARLY) {
            uint32_t x0, x1, x2;
            split3(sc, x0, x1, x2);
            // slots 0..7: x0 x0 x0 x1 | x1 x2 0 0 (paired with y0 y1 y2 y0 | y1 y0 0 0)
            d.ta[0][ht] = make_uint2(x0 | (x0 << 16), x0 | (x1 << 16));
            d.ta[1][ht] = make_uint2(x1 | (x2 << 16), 0);
        } else if (has_scale) {
            uint32_t y0, y1, y2;
            split3(sc, y0, y1, y2);
            d.tb[0][ht] = make_uint2(y0 | (y1 << 16), y2 | (y0 << 16));
            d.tb[1][ht] = make_uint2(y1 | (y0 << 16), 0);
        }
    };

    float acc[2][2][16];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mt][nt][r] = 0.0f;

    const int trow = lane & 31, thalf = lane >> 5;
    auto tile_mt = [](int i) { return i >> 1; };
    auto tile_nt = [](int i) { return (i ^ (i >> 1)) & 1; };

    v16f P[2] = {v16f{}, v16f{}};
    v16f S[2] = {v16f{}, v16f{}};
    auto fold_quarter = [&](const v16f& p, const v16f& s, int mt, int nt, int q) {
        float* c = &acc[mt][nt][4 * q];
#pragma unroll
        for (int r = 0; r < 4; ++r) c[r] = fmaf(s[4 * q + r], p[4 * q + r], c[r]);
        anchor4(c[0], c[1], c[2], c[3]);
    };
    auto debug_tile = [&](const v16f& p, int mt, int nt, int j) {
        if (DEBUG_P) {
            const int n = n0 + wn * 64 + nt * 32 + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm * 64 + mt * 32 + acc_row(r, lane);
                if (m < a.M && n < a.N)
                    if (int32_t* dp = psum_at(a.psum, a.prows, m, n, a.N, a.G, j)) *dp = (int)p[r];
            }
        }
    };

    // Every wave waits for its own direct-to-LDS loads of the next stage
    // (issued a stage ago; only the next stage's loads, MY_LOADS + 1
    // operations, stay in flight) before the barrier, so that after it every
    // wave's copies of the next stage have landed.
    auto wait_copies = [&]() {
        if (EARLY) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
    };
    static_assert(LOADS == 36, "wait_copies counts 5 (waves 0..3) or 4 loads per wave and stage, plus the scale");

    // the scale of stage t + 1 (loaded a stage ago), written into its buffer
    // during stage t
    float s_next;

    // one stage t out of buffer d (stage t + 1's scales go to buffer dn,
    // stage t + 2's rows to buffer dc)
    auto stage = [&](int t, StageBuf& d, StageBuf& dn, StageBuf& dc) {
        // scale operands first (the first instruction of every window uses
        // them), then the fragments, three chunks per lane and tile (both
        // K-steps): those of tile 0 here, B of tile 1 in window 0, A of
        // tiles 2-3 in window 1, so that the reads right after the barrier
        // (all waves at once) are few and the rest overlap the MFMAs
        uint4 fa[2][3], fb[2][3];
        v4s opa[2], opb[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            opa[i] = __builtin_bit_cast(v4s, d.ta[thalf][wm * 64 + 32 * i + trow]);
            opb[i] = __builtin_bit_cast(v4s, d.tb[thalf][wn * 64 + 32 * i + trow]);
        }
#pragma unroll
        for (int c = 0; c < 3; ++c) {
            fa[0][c] = d.a[3 * thalf + c][wm * 64 + trow];
            fb[0][c] = d.b[3 * thalf + c][wn * 64 + trow];
        }
        // stage t + 2 in flight (its buffer was last read in stage t - 1)
        copy_stage(dc, t + 2);
        const float s_new = load_scale(t + 2);
        fence_sched();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int mt = tile_mt(i), nt = tile_nt(i);
            const int pi = (i + 3) & 3;
            const int pmt = tile_mt(pi), pnt = tile_nt(pi);
            v16f& Pc = P[i & 1];
            v16f& Pp = P[(i + 1) & 1];
            v16f& Sp = S[(i + 1) & 1];
            anchor16(Pp);
            anchor16(Sp);
            // This tile's first K-step, its scale product (folded in the next
            // window), its second K-step: the second depends on the first,
            // so the scale product goes between them.  Then the previous
            // tile's fold.
            Pc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(step_operand(fa[mt], 0), step_operand(fb[nt], 0),
                                                                 v16f{}, FMT_FP6, FMT_FP6, 0, SCALE_E8M0, 0,
                                                                 SCALE_E8M0);
            if (i == 0)
#pragma unroll
                for (int c = 0; c < 3; ++c) fb[1][c] = d.b[3 * thalf + c][wn * 64 + 32 + trow];
            if (i == 1)
#pragma unroll
                for (int c = 0; c < 3; ++c) fa[1][c] = d.a[3 * thalf + c][wm * 64 + 32 + trow];
            fence_sched();
            S[i & 1] = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(opa[mt], opb[nt], v16f{}, 0, 0, 0);
            fence_sched();
            Pc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(step_operand(fa[mt], 1), step_operand(fb[nt], 1),
                                                                 Pc, FMT_FP6, FMT_FP6, 0, SCALE_E8M0, 0, SCALE_E8M0);
            anchor16(Pc);
            fence_sched();
            fold_quarter(Pp, Sp, pmt, pnt, 0);
            fold_quarter(Pp, Sp, pmt, pnt, 1);
            fold_quarter(Pp, Sp, pmt, pnt, 2);
            fold_quarter(Pp, Sp, pmt, pnt, 3);
            if (DEBUG_P && (i > 0 || t > 0)) debug_tile(Pp, pmt, pnt, i == 0 ? s0 + t - 1 : s0 + t);
            if (i == 3) store_scale(dn, s_next);
            fence_sched();
        }
        s_next = s_new;
        wait_copies();
        lds_barrier();
    };

    // --- prologue: stages 0 and 1 in flight (rows straight to LDS, scales
    // through registers), stage 0's scales into buffer 0 ---
    copy_stage(b0, 0);
    const float s_first = load_scale(0);
    copy_stage(b1, 1);
    s_next = load_scale(1);
    store_scale(b0, s_first);
    wait_copies();
    lds_barrier();

    // stage t reads buffer t % 3: the loop is unrolled by three so that the
    // buffers are compile-time objects (distinct LDS variables, so that the
    // compiler's wait analysis can tell a buffer being read from the ones
    // being filled)
    for (int t0 = 0; t0 < stages; t0 += 3) {
        stage(t0, b0, b1, b2);
        if (t0 + 1 < stages) stage(t0 + 1, b1, b2, b0);
        if (t0 + 2 < stages) stage(t0 + 2, b2, b0, b1);
    }
    // the copies past the last stage are still in flight: let them land
    // before the workgroup's LDS can be handed to another one
    __builtin_amdgcn_s_waitcnt(0);
    // the last tile of the last stage
#pragma unroll
    for (int q = 0; q < 4; ++q) fold_quarter(P[1], S[1], tile_mt(3), tile_nt(3), q);
    debug_tile(P[1], tile_mt(3), tile_nt(3), s0 + stages - 1);

    if (a.part) {
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
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const int n = n0 + wn * 64 + nt * 32 + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm * 64 + mt * 32 + acc_row(r, lane);
                if (m < a.M && n < a.N) {
                    float v = acc[mt][nt][r];
                    asm volatile("" : "+v"(v));
                    const int64_t o = (int64_t)m * a.N + n;
                    a.y16[o] = (_Float16)v;
                    if (a.y32) a.y32[o] = v;
                }
            }
        }
}

template <bool DEBUG_P>
__global__ __launch_bounds__(THREADS, 1) void gemm_f6_kernel(F6Args a)
{
    __shared__ StageBuf b0, b1, b2;
    if (__builtin_amdgcn_readfirstlane(threadIdx.x) < HALF)
        f6_body<DEBUG_P, true>(a, b0, b1, b2);
    else
        f6_body<DEBUG_P, false>(a, b0, b1, b2);
}

// Y of the K-split tiles: the parts' sums added in part order
__global__ __launch_bounds__(256) void f6_split_reduce_kernel(F6Args a)
{
    const int idx = blockIdx.x * 256 + threadIdx.x;
    constexpr int PER_TILE = BM * BN / 4;
    if (idx >= a.ntail * PER_TILE) return;
    const int lin = idx / PER_TILE, rem = idx - lin * PER_TILE;
    const int row = rem / (BN / 4), col = (rem - row * (BN / 4)) * 4;
    int by, bx;
    tile_coords(a, a.tile0 + lin, by, bx);
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
            float v = s[j];
            asm volatile("" : "+v"(v));
            const int64_t o = (int64_t)m * a.N + n;
            a.y16[o] = (_Float16)v;
            if (a.y32) a.y32[o] = v;
        }
    }
}

void launch_f6(const F6Args& t, int grid, hipStream_t stream)
{
    if (t.psum) gemm_f6_kernel<true><<<grid, THREADS, 0, stream>>>(t);
    else gemm_f6_kernel<false><<<grid, THREADS, 0, stream>>>(t);
}

}  // namespace

bool f6_supports(const GemmProblem& p)
{
    // 32-bit buffer offsets within one workgroup's row blocks
    const uint64_t block_bytes = (uint64_t)p.K / KSTAGE * TILE_BYTES;
    return p.K % KSTAGE == 0 && block_bytes * (BM / 64) < (1ull << 31) && (uint64_t)p.K / KSTAGE * 4 * BM < (1ull << 31);
}

hipError_t launch_gemm_f6(const GemmProblem& p, hipStream_t stream)
{
    F6Args t{};
    t.qa = p.qa;
    t.sa = p.sa;
    t.qw = p.qw;
    t.sw = p.sw;
    t.M = p.M;
    t.N = p.N;
    t.K = p.K;
    t.G = p.K / KSTAGE;
    t.y16 = static_cast<_Float16*>(p.y16);
    t.y32 = p.y32;
    t.psum = p.psum;
    t.prows = p.prows;
    t.tiles_m = (p.M + BM - 1) / BM;
    t.tiles_n = (p.N + BN - 1) / BN;
    t.group_m = t.tiles_m < 4 ? t.tiles_m : 4;   // one XCD's 32 tiles in flight: 4 x 8 blocks
    t.nparts = 1;
    // the partial last round as K parts: the split (and workspace) of the
    // nibble kernels for groups of 128
    GemmProblem g = p;
    g.ga = g.gw = KSTAGE;
    PingpongSplit sp = pingpong_split(g);
    if (sp.tail && (!p.ws || p.ws_bytes < sp.bytes)) sp.tail = 0;
    if (sp.tail == 0) {
        launch_f6(t, sp.tiles, stream);
        return hipGetLastError();
    }
    if (sp.tiles > sp.tail) launch_f6(t, sp.tiles - sp.tail, stream);
    F6Args k = t;
    k.tile0 = sp.tiles - sp.tail;
    k.ntail = sp.tail;
    k.nparts = sp.nparts;
    k.part = static_cast<float*>(p.ws);
    launch_f6(k, sp.nparts * sp.tail, stream);
    f6_split_reduce_kernel<<<(sp.tail * (BM * BN / 4) + 255) / 256, 256, 0, stream>>>(k);
    return hipGetLastError();
}

}  // namespace apex4
