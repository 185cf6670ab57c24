// W4A4 GEMM for 17..64 token rows (decode with a batch of sequences) on
// gfx950: weight rows streamed through LDS by direct loads, as in the
// LDS-streaming kernel for up to 16 rows, with K walked outside the output
// column blocks so that the activations of a K item are loaded once and serve
// several blocks.
//
// Why the order matters.  At 64 rows the activation bytes of a K item are four
// times the weight bytes of one 16-column block.  Walking the blocks inside the
// K items lets a workgroup bring the item's activation rows into LDS once and
// reuse them for BG blocks (2, 4 or, with up to 32 rows, 8), whose fp32
// accumulators stay in registers until the last item.
//
// Work split.  Output columns come in blocks of 16 (16 weight rows, one
// v_mfma_i32_16x16x64_i8 column tile); the blocks are dealt round-robin to the
// workgroups (one per CU) and each workgroup takes its blocks BG at a time (a
// group).  An item is 1024 K values (512 bytes of a row: loads of whole
// 512-byte row pieces stream at ~5.1 TB/s here, 1 KB pieces at ~5.2).  A unit
// is one (block, item) pair.  Units run group by group, item by item, block by
// block; their weight pieces and weight scales land in 8 LDS buffers, 7 units
// ahead.  Each item's activation rows (MT x 16 rows x 512 bytes) and s_a come
// into one of two LDS buffers at the first unit of the item before.  The
// barrier of an item's first unit waits for them, so only the copies issued
// after them (BG units' worth, at most 6) stay in flight there; the other
// barriers leave the copies of the 6 later units in flight.  Every LDS access
// in the loop is inline asm with its own wait: the compiler's wait analysis
// cannot always tell the direct-to-LDS copies into different buffers apart and
// would drain them.
//
// K split.  With at most 2 column blocks per workgroup (e.g. N = 8192: 512
// blocks on 256 CUs) an item's activation rows serve only 2 blocks' weights.
// Then (groups of 128) the workgroups form two sets, each walking half of K
// over twice the blocks; their fp32 results go to the caller's workspace and
// a small kernel adds the two halves in a fixed order.
//
// Each of the 8 waves owns 128 K values of every item, i.e. one group of 128:
// two K-steps per row tile.  Its activation fragments and s_a for the item are
// read from LDS once, at the item's first unit.  At the end of a group the
// waves' partial tiles of each block are added in a fixed order through LDS
// (the buffer of the finished item's activations).
//
// LDS row pieces are swizzled: the 16-byte chunk c of a row r sits at slot
// c ^ (r mod 16), so the 16 rows' fragment reads of one chunk hit different
// banks.  Lane (row i, block kb) takes chunk 4w + kb of its row: the first 8
// bytes feed K-step 0, the last 8 K-step 1, both operands alike.  Widening as
// in the other MFMA kernels: (w << 4) & 0xF0F0F0F0 and w & 0xF0F0F0F0 give
// 16*c, the MFMA returns 256*P exactly and 2^-8 is applied to the finished
// sums.
#include "internal.h"

namespace apex4 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int ROWS = 16;                 // weight rows per block
constexpr int IK = 1024;                 // K values per item
constexpr int PIECE = IK / 2;            // 512 packed bytes per row and item
constexpr int WAVES = 8;
constexpr int THREADS = WAVES * 64;
constexpr uint32_t OOB = 0x80000000u;    // past every buffer: reads zeros

struct KouterArgs {
    const uint8_t* qa;
    const float* sa;
    const uint8_t* qw;
    const float* sw;
    int M, N, K;
    int Ga, Gw;        // scale columns per row: K/ga, K/gw
    int G;             // K / gs
    int blocks;        // ceil(N / 16)
    int items;         // ceil(K / 1024)
    _Float16* y16;
    float* y32;
    int32_t* psum;
    PsumRows prows;
    // K split (groups of 128): the workgroups come in kparts equal sets, set q
    // walking items [q items / kparts, (q+1) items / kparts) of its blocks
    // (dealt round-robin within the set) and writing its fp32 results to
    // part[q] ([M][N]) for the reduction kernel; kparts = 1: no split.
    int kparts;
    float* part;
};

// LDS: NBUF unit buffers (16 weight-row pieces, then s_w in 8 regions of 64
// floats: regions 0 and 1 hold rows 0-7 and 8-15 as [row][8 groups], the
// other waves' copies repeat them), two activation buffers by item parity (up
// to 64 rows x 512 bytes; also the reduction tile), two s_a buffers ([8
// groups][64 rows]).
constexpr int UNIT_W = ROWS * PIECE;
constexpr int UNIT_BYTES = UNIT_W + WAVES * 256;
constexpr int NBUF_MAX = 8;
constexpr int ACT_BYTES = 64 * PIECE;
__shared__ __attribute__((aligned(16))) uint8_t lds_units[NBUF_MAX * UNIT_BYTES];
__shared__ __attribute__((aligned(16))) uint8_t lds_act[2][ACT_BYTES];
__shared__ __attribute__((aligned(16))) float lds_sa[2][8 * 64];

__device__ inline __amdgpu_buffer_rsrc_t buffer_of(const void* p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

__device__ inline uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(const lds_void*)p; }

// Inline-asm LDS accesses, each read block with its own wait (see the file
// comment).
__device__ inline void lds_read_w(uint32_t a0, uint32_t s0a, uint4& w0, float& s0)
{
    v4i r0;
    asm volatile("ds_read_b128 %0, %2\n\t"
                 "ds_read_b32 %1, %3\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(r0), "=&v"(s0)
                 : "v"(a0), "v"(s0a)
                 : "memory");
    w0 = __builtin_bit_cast(uint4, r0);
}

__device__ inline v4i lds_read16(uint32_t a)
{
    v4i r;
    asm volatile("ds_read_b128 %0, %1\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(r)
                 : "v"(a)
                 : "memory");
    return r;
}

__device__ inline float lds_read_f(uint32_t a)
{
    float v;
    asm volatile("ds_read_b32 %0, %1\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(v)
                 : "v"(a)
                 : "memory");
    return v;
}

// the 8 waves' partial values of one tile element, STRIDE bytes apart
template <int STRIDE>
__device__ inline void lds_read_red(uint32_t ra, float (&v)[WAVES])
{
    asm volatile("ds_read_b32 %0, %8\n\t"
                 "ds_read_b32 %1, %8 offset:%9\n\t"
                 "ds_read_b32 %2, %8 offset:%10\n\t"
                 "ds_read_b32 %3, %8 offset:%11\n\t"
                 "ds_read_b32 %4, %8 offset:%12\n\t"
                 "ds_read_b32 %5, %8 offset:%13\n\t"
                 "ds_read_b32 %6, %8 offset:%14\n\t"
                 "ds_read_b32 %7, %8 offset:%15\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]),
                   "=&v"(v[7])
                 : "v"(ra), "i"(STRIDE), "i"(2 * STRIDE), "i"(3 * STRIDE), "i"(4 * STRIDE), "i"(5 * STRIDE),
                   "i"(6 * STRIDE), "i"(7 * STRIDE)
                 : "memory");
}

__device__ inline void lds_write16(uint32_t p, v4f v)
{
    asm volatile("ds_write_b128 %0, %1" : : "v"(p), "v"(v) : "memory");
}

__device__ inline v4i widen_lo(uint4 w)
{
    return v4i{(int)((w.x << 4) & 0xF0F0F0F0u), (int)(w.x & 0xF0F0F0F0u),
               (int)((w.y << 4) & 0xF0F0F0F0u), (int)(w.y & 0xF0F0F0F0u)};
}

__device__ inline v4i widen_hi(uint4 w)
{
    return v4i{(int)((w.z << 4) & 0xF0F0F0F0u), (int)(w.z & 0xF0F0F0F0u),
               (int)((w.w << 4) & 0xF0F0F0F0u), (int)(w.w & 0xF0F0F0F0u)};
}

constexpr int waitcnt(int vm, int lgkm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8); }

// an LDS-only barrier (the direct copies in flight stay in flight)
__device__ inline void lds_barrier()
{
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(waitcnt(63, 0));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// GM: 1 (groups of 128), 0 (one group over K).  MIXED: per-channel weight
// scales, activation groups of 128.  MT: 16-row tiles of M (2 or 4).  BG:
// blocks per group (2, 4 or 8).
template <int GM, bool MIXED, bool DEBUG_P, int MT, int BG>
__global__ __launch_bounds__(THREADS) void gemm_kouter_kernel(KouterArgs a)
{
    constexpr int NBUF = NBUF_MAX;
    constexpr int VM_UNIT = 2;                             // vector memory operations per wave and unit
    constexpr bool SW_PER_GROUP = GM == 1 && !MIXED;       // s_w varies along K
    constexpr bool SA_PER_GROUP = GM == 1;                 // s_a varies along K
    constexpr int GPI = IK / 128;                          // groups per item (GM 1)
    constexpr int RED_STRIDE = 64 * MT * 16;               // bytes between two waves' partial tiles
    static_assert(NBUF <= NBUF_MAX && WAVES * RED_STRIDE <= ACT_BYTES, "LDS");
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t rowbytes = (uint32_t)a.K / 2;
    // this workgroup's set (K part) and its index within the set
    const int wgs = gridDim.x / a.kparts;
    const int kq = blockIdx.x / wgs, wid = blockIdx.x - kq * wgs;
    const int item0 = kq * a.items / a.kparts;
    const int nit = (kq + 1) * a.items / a.kparts - item0;    // items walked
    const int nb = wid < a.blocks ? (a.blocks - 1 - wid) / wgs + 1 : 0;
    const int ngroups = (nb + BG - 1) / BG;
    const int n_items = ngroups * nit;                     // (group, item) pairs
    const int total = n_items * BG;                        // units
    const __amdgpu_buffer_rsrc_t rW = buffer_of(a.qw, (uint32_t)a.N * rowbytes);
    const __amdgpu_buffer_rsrc_t rA = buffer_of(a.qa, (uint32_t)a.M * rowbytes);
    const __amdgpu_buffer_rsrc_t rS = buffer_of(a.sw, (uint32_t)a.N * a.Gw * 4);
    const __amdgpu_buffer_rsrc_t rSA = buffer_of(a.sa, (uint32_t)a.M * a.Ga * 4);
    const int fi = lane & 15, fkb = lane >> 4;             // fragment row, K block
    const int m_out = 4 * fkb;                             // output rows m_out..m_out+3 of a row tile
    const int slot_k = (4 * wave + fkb) ^ fi;              // LDS slot of this lane's chunk of row fi

    // unit u: group u / (nit * BG), item item0 + (u / BG) % nit, block slot u % BG
    auto unit_block = [&](int u, int& b, int& it, bool& live) {
        const int ii = u / BG, j = u - ii * BG;
        const int grp = ii / nit;
        it = item0 + ii - grp * nit;
        const int slot = grp * BG + j;
        live = u < total && slot < nb;
        b = wid + wgs * slot;
    };

    // --- copy of unit u into buffer bi: weight rows 2w (lanes 0-31) and
    // 2w+1 (lanes 32-63), lane l fetching chunk (l mod 32) ^ r of row r; s_w
    // of rows 8(w & 1)..8(w & 1)+7 (lane l: row l >> 3, group l & 7) ---
    auto copy_unit = [&](int bi, int u) {
        int b, it;
        bool live;
        unit_block(u, b, it, live);
        uint8_t* d = lds_units + bi * UNIT_BYTES;
        {
            const int r = 2 * wave + (lane >> 5);
            const uint32_t pos = (uint32_t)it * PIECE + 16 * ((lane & 31) ^ r);
            const bool in = live && pos < rowbytes;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rW, (lds_void*)(d + 2 * wave * PIECE), 16,
                                                     in ? (int)((uint32_t)(b * ROWS + r) * rowbytes + pos) : (int)OOB,
                                                     0, 0, 0);
        }
        const int n = b * ROWS + 8 * (wave & 1) + (lane >> 3), gi = lane & 7;
        const int g = SW_PER_GROUP ? it * GPI + gi : 0;
        const bool in = live && n < a.N && (SW_PER_GROUP ? g < a.Gw : gi == 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rS, (lds_void*)(d + UNIT_W + 256 * wave), 4,
                                                 in ? (int)(((uint32_t)n * a.Gw + g) * 4) : (int)OOB, 0, 0, 0);
    };

    // --- activation rows and s_a of (group, item) ii into buffers ii & 1:
    // row pairs w, w + 8, ... (lanes 0-31 and 32-63, the same swizzle), and
    // group w of the item's s_a (lane l: row l) ---
    auto load_item = [&](int ii) {
        const bool live = ii < n_items;
        const int it = item0 + (live ? ii % nit : 0);
        uint8_t* d = lds_act[ii & 1];
#pragma unroll
        for (int k = 0; k < MT; ++k) {
            const int pr = wave + WAVES * k, r = 2 * pr + (lane >> 5);
            const uint32_t pos = (uint32_t)it * PIECE + 16 * ((lane & 31) ^ (r & 15));
            const bool in = live && r < a.M && pos < rowbytes;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_void*)(d + 2 * pr * PIECE), 16,
                                                     in ? (int)((uint32_t)r * rowbytes + pos) : (int)OOB, 0, 0, 0);
        }
        const int g = SA_PER_GROUP ? it * GPI + wave : 0;
        const bool in = live && lane < a.M && (SA_PER_GROUP ? g < a.Ga : wave == 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rSA, (lds_void*)(&lds_sa[ii & 1][64 * wave]), 4,
                                                 in ? (int)(((uint32_t)lane * a.Ga + g) * 4) : (int)OOB, 0, 0, 0);
    };

    // the first item's activations, then the first NBUF - 1 units
    load_item(0);
#pragma unroll
    for (int i = 0; i < NBUF - 1; ++i) copy_unit(i, i);

    v4i aw[MT][2];                                         // widened activation fragments: [tile][K step]
    v4f sa4[MT];                                           // s_a of rows m_out..m_out+3 of each tile
    float acc[BG][MT][4];
    v4i pk[BG][MT];                                        // one group over K: exact int32 sums
    float swk[BG];                                         // one group or mixed: s_w of the lane's column
#pragma unroll
    for (int j = 0; j < BG; ++j) {
        swk[j] = 0.0f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            pk[j][mt] = v4i{};
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[j][mt][r] = 0.0f;
        }
    }
    int opaque_zero;                                       // zero, unknown to the compiler
    asm volatile("v_mov_b32 %0, 0" : "=v"(opaque_zero));

    // Finish the group that ends with item ii: per block, the waves' partial
    // tiles go to LDS (the item's activation buffer, whose reads all ended
    // before the last unit's barrier), then thread (w, l) adds the 8 partials
    // of column l & 15, (tile, register) pairs 2w and 2w + 1 (MT = 4) or w
    // (MT = 2), in wave order, and stores them.
    auto finish_group = [&](int ii) {
        const int grp = ii / nit;
        float* red = reinterpret_cast<float*>(lds_act[ii & 1]);
        const float* sab = lds_sa[ii & 1];
#pragma unroll
        for (int j = 0; j < BG; ++j) {
            const int slot = grp * BG + j;
            const int b = wid + wgs * slot;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const uint32_t p = lds_addr(&red[((wave * 64 + lane) * MT + mt) * 4]);
                if (GM == 0) {
                    // (an ordinary vector instruction reads the MFMA result
                    // first, so the compiler puts the result latency before it)
                    const v4i pv = pk[j][mt] ^ opaque_zero;
                    lds_write16(p, __builtin_bit_cast(v4f, pv));
                } else {
                    lds_write16(p, v4f{acc[j][mt][0], acc[j][mt][1], acc[j][mt][2], acc[j][mt][3]});
                }
            }
            lds_barrier();
            if (slot < nb) {
#pragma unroll
                for (int e = 0; e < (MT == 4 ? 2 : 1); ++e) {
                    const int pr = (MT == 4 ? 2 * wave + e : wave);   // (tile, register) pair
                    const int mt = pr >> 2, r = pr & 3;
                    const int m = 16 * mt + 4 * (lane >> 4) + r, n = b * ROWS + (lane & 15);
                    float v8[WAVES];
                    lds_read_red<RED_STRIDE>(lds_addr(&red[(lane * MT + mt) * 4 + r]), v8);
                    float v;
                    if (GM == 0) {
                        int p = 0;
#pragma unroll
                        for (int w = 0; w < WAVES; ++w) p += __builtin_bit_cast(int, v8[w]);
                        const float s_a0 = lds_read_f(lds_addr(&sab[m]));
                        const float S = s_a0 * 0.00390625f * swk[j];
                        v = S * (float)p;
                        if (DEBUG_P && m < a.M && n < a.N)
                            if (int32_t* d = psum_at(a.psum, a.prows, m, n, a.N, 1, 0)) *d = p >> 8;
                    } else {
                        v = 0.0f;
#pragma unroll
                        for (int w = 0; w < WAVES; ++w) v += v8[w];
                        v *= 0.00390625f;                // the widening's 2^8, exactly
                        if (MIXED) v *= swk[j];
                    }
                    asm volatile("" : "+v"(v));   // y16 is the fp16 rounding of y32
                    if (m < a.M && n < a.N) {
                        const int64_t off = (int64_t)m * a.N + n;
                        if (a.part) {
                            a.part[(int64_t)kq * a.M * a.N + off] = v;
                        } else {
                            a.y16[off] = (_Float16)v;
                            if (a.y32) a.y32[off] = v;
                        }
                    }
                }
            }
            lds_barrier();
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                pk[j][mt] = v4i{};
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[j][mt][r] = 0.0f;
            }
        }
    };

    // Unit u uses buffer u % NBUF (a run-time choice: every LDS access below
    // takes a computed address); the loop is unrolled by BG so that the block
    // slot, the accumulators and the item start are compile-time.
    for (int u0 = 0; u0 < total; u0 += BG)
#pragma unroll
    for (int j = 0; j < BG; ++j) {
        const int u = u0 + j;
        const int ii = u0 / BG;
        // unit u has landed (the copies of the NBUF - 2 later units stay in
        // flight), and every wave is done with unit u - 1, whose buffer the
        // copy of u + NBUF - 1 reuses.  At an item's first unit the item's
        // activation copies, issued BG units ago, must have landed too: only
        // the copies of the BG units issued after them may stay in flight.
        constexpr int J0_WAIT = VM_UNIT * (BG < NBUF - 2 ? BG : NBUF - 2);
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("" ::: "memory");
        if (j == 0)
            __builtin_amdgcn_s_waitcnt(waitcnt(J0_WAIT, 0));
        else
            __builtin_amdgcn_s_waitcnt(waitcnt(VM_UNIT * (NBUF - 2), 0));
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        if (j == 0) {
            // this item's activation fragments and s_a; then the next item's
            // copies (into the other buffers, last read by item ii - 1)
            const uint8_t* act = lds_act[ii & 1];
            const float* sab = lds_sa[ii & 1];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const uint4 x = __builtin_bit_cast(uint4, lds_read16(lds_addr(act + (16 * mt + fi) * PIECE + 16 * slot_k)));
                aw[mt][0] = widen_lo(x);
                aw[mt][1] = widen_hi(x);
                if (GM == 1) sa4[mt] = __builtin_bit_cast(v4f, lds_read16(lds_addr(&sab[64 * wave + 16 * mt + m_out])));
            }
            load_item(ii + 1);
        }
        copy_unit((u + NBUF - 1) % NBUF, u + NBUF - 1);

        int b, it;
        bool live;
        unit_block(u, b, it, live);
        const uint8_t* cur = lds_units + (u % NBUF) * UNIT_BYTES;
        const float* csw = reinterpret_cast<const float*>(cur + UNIT_W);
        // weight fragment: chunk 4w + kb of row fi; s_w of column fi for the
        // wave's group (group 0: one group over K or mixed)
        uint4 w0;
        float sw0;
        lds_read_w(lds_addr(cur + fi * PIECE + 16 * slot_k),
                   lds_addr(&csw[64 * (fi >> 3) + 8 * (fi & 7) + (SW_PER_GROUP ? wave : 0)]), w0, sw0);
        if (GM == 0 || MIXED) swk[j] = sw0;
        const v4i wl = widen_lo(w0), wh = widen_hi(w0);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            if (GM == 0) {
                const v4i c = __builtin_amdgcn_mfma_i32_16x16x64_i8(aw[mt][0], wl, pk[j][mt], 0, 0, 0);
                pk[j][mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aw[mt][1], wh, c, 0, 0, 0);
                continue;
            }
            v4i P = __builtin_amdgcn_mfma_i32_16x16x64_i8(aw[mt][0], wl, v4i{}, 0, 0, 0);
            P = __builtin_amdgcn_mfma_i32_16x16x64_i8(aw[mt][1], wh, P, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float S = MIXED ? sa4[mt][r] : sa4[mt][r] * sw0;
                acc[j][mt][r] = fmaf(S, (float)P[r], acc[j][mt][r]);
            }
            if (DEBUG_P) {
                const int gj = it * GPI + wave, n = b * ROWS + fi;
                if (live && gj < a.G) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int m = 16 * mt + m_out + r;
                        if (m < a.M && n < a.N)
                            if (int32_t* d = psum_at(a.psum, a.prows, m, n, a.N, a.G, gj)) *d = P[r] >> 8;
                    }
                }
            }
        }
        if (j == BG - 1 && it == item0 + nit - 1) finish_group(ii);
    }
    __builtin_amdgcn_s_waitcnt(waitcnt(0, 0));
}

// Y = the K parts' results added in part order (fp16 the RNE rounding of the
// fp32 sum); 4 consecutive outputs per thread, read as 16-byte vectors when
// M*N is a multiple of 4 (then every part starts 16-byte aligned)
__global__ __launch_bounds__(256) void kouter_split_reduce_kernel(KouterArgs a)
{
    const int64_t mn = (int64_t)a.M * a.N;
    const int64_t i0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i0 >= mn) return;
    float v[4];
    if ((mn & 3) == 0) {
        float4 p = *reinterpret_cast<const float4*>(a.part + i0);
        v[0] = p.x, v[1] = p.y, v[2] = p.z, v[3] = p.w;
        for (int q = 1; q < a.kparts; ++q) {
            p = *reinterpret_cast<const float4*>(a.part + q * mn + i0);
            v[0] += p.x, v[1] += p.y, v[2] += p.z, v[3] += p.w;
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[e] = 0.0f;
            if (i0 + e < mn) {
                v[e] = a.part[i0 + e];
                for (int q = 1; q < a.kparts; ++q) v[e] += a.part[q * mn + i0 + e];
            }
        }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if (i0 + e < mn) {
            float x = v[e];
            asm volatile("" : "+v"(x));
            a.y16[i0 + e] = (_Float16)x;
            if (a.y32) a.y32[i0 + e] = x;
        }
    }
}

// workgroups: one per block up to 256, in kparts equal sets
int kouter_grid(const KouterArgs& s)
{
    const int want = s.blocks * s.kparts;
    const int g = want < 256 ? want : 256;
    return g - g % s.kparts;
}

template <int GM, bool MIXED, int MT, int BG>
hipError_t launch_g(const KouterArgs& s, bool dbg, hipStream_t stream)
{
    const int grid = kouter_grid(s);
    if (dbg) gemm_kouter_kernel<GM, MIXED, true, MT, BG><<<grid, THREADS, 0, stream>>>(s);
    else gemm_kouter_kernel<GM, MIXED, false, MT, BG><<<grid, THREADS, 0, stream>>>(s);
    if (s.kparts > 1) {
        const int64_t mn = (int64_t)s.M * s.N;
        kouter_split_reduce_kernel<<<(unsigned)((mn + 1023) / 1024), 256, 0, stream>>>(s);
    }
    return hipGetLastError();
}

// blocks per group: 2, 4 or 8 (4 row tiles: at most 4, for the registers)
template <int GM, bool MIXED, int MT>
hipError_t launch_mt(const KouterArgs& s, bool dbg, hipStream_t stream)
{
    const int wgs = kouter_grid(s) / s.kparts;
    const int per_wg = (s.blocks + wgs - 1) / wgs;
    if (per_wg <= 2) return launch_g<GM, MIXED, MT, 2>(s, dbg, stream);
    if (per_wg <= 4 || MT == 4) return launch_g<GM, MIXED, MT, 4>(s, dbg, stream);
    return launch_g<GM, MIXED, MT, MT == 4 ? 4 : 8>(s, dbg, stream);
}

template <int GM, bool MIXED>
hipError_t launch_mode(const KouterArgs& s, bool dbg, hipStream_t stream)
{
    if (s.M <= 32) return launch_mt<GM, MIXED, 2>(s, dbg, stream);
    return launch_mt<GM, MIXED, 4>(s, dbg, stream);
}

}  // namespace

int kouter_kparts(const GemmProblem& p)
{
    // Two K parts when a workgroup would get at most 2 column blocks (groups
    // of 128 only, at least 2 items per part): each workgroup then walks half
    // the items over twice the blocks, so each item's activation rows serve
    // twice the weight bytes (and with fewer than 256 blocks, twice the CUs
    // work).  One group over K keeps its single rounding.
    const int gs = p.ga < p.gw ? p.ga : p.gw;
    const int blocks = (p.N + ROWS - 1) / ROWS, items = (p.K + IK - 1) / IK;
    const int grid = blocks < 256 ? blocks : 256;
    if (gs != 128 || items < 4 || (blocks + grid - 1) / grid > 2) return 1;
    return 2;
}

size_t kouter_workspace_bytes(const GemmProblem& p)
{
    const int kp = kouter_kparts(p);
    return kp > 1 ? (size_t)kp * p.M * p.N * sizeof(float) : 0;
}

bool kouter_supports(const GemmProblem& p)
{
    if (p.M < 17 || p.M > 64 || p.K % 128 != 0) return false;
    const int gs = p.ga < p.gw ? p.ga : p.gw;
    const bool mixed = p.gw == p.K && p.ga != p.gw;
    // groups of 128 (a wave's K slice of an item), one group over K, or mixed
    // with activation groups of 128
    if (mixed) {
        if (p.ga != 128) return false;
    } else if (p.ga != p.gw || !(gs == 128 || gs == p.K)) {
        return false;
    }
    // 32-bit buffer offsets
    const uint64_t wbytes = (uint64_t)p.N * (p.K / 2), sbytes = (uint64_t)p.N * (p.K / p.gw) * 4;
    return wbytes < OOB && sbytes < OOB && (uint64_t)p.M * (p.K / 2) < OOB && (uint64_t)p.M * (p.K / p.ga) * 4 < OOB;
}

hipError_t launch_gemm_kouter(const GemmProblem& p, hipStream_t stream)
{
    KouterArgs s;
    s.qa = p.qa;
    s.sa = p.sa;
    s.qw = p.qw;
    s.sw = p.sw;
    s.M = p.M;
    s.N = p.N;
    s.K = p.K;
    s.Ga = p.K / p.ga;
    s.Gw = p.K / p.gw;
    const int gs = p.ga < p.gw ? p.ga : p.gw;
    s.G = p.K / gs;
    s.blocks = (p.N + ROWS - 1) / ROWS;
    s.items = (p.K + IK - 1) / IK;
    s.y16 = static_cast<_Float16*>(p.y16);
    s.y32 = p.y32;
    s.psum = p.psum;
    s.prows = p.prows;
    s.kparts = kouter_kparts(p);
    s.part = static_cast<float*>(p.ws);
    // the split needs its workspace (each half writes the debug sums of its
    // own groups)
    if (s.kparts > 1 && (!p.ws || p.ws_bytes < kouter_workspace_bytes(p))) s.kparts = 1;
    if (s.kparts == 1) s.part = nullptr;
    const bool mixed = p.gw == p.K && p.ga != p.gw;
    const bool dbg = p.psum != nullptr;
    if (mixed) return launch_mode<1, true>(s, dbg, stream);
    if (gs == p.K && gs != 128) return launch_mode<0, false>(s, dbg, stream);   // (K = 128: one group of 128)
    return launch_mode<1, false>(s, dbg, stream);
}

}  // namespace apex4
