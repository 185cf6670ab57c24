// W4A4 GEMM for up to 16 token rows (decode) on gfx950: weight rows streamed
// through LDS in 1 KB row pieces, int8 MFMA on the widened nibbles.
//
// A decode GEMM is bound by reading the packed weights once.  On this chip the
// access pattern decides how close that gets to the HBM rate: loads that cover
// 1 KB of one row per instruction stream a decode-sized matrix at ~6 TB/s,
// where 64-byte pieces of 16 rows per instruction (the shape a matrix
// operand wants) reach ~3.7 TB/s.  So the weights (and the activation rows)
// come in through direct global -> LDS loads of whole 1 KB row pieces, and
// the MFMA fragments are read from LDS.
//
// Work split.  Output columns come in blocks of 16 (16 weight rows); the
// blocks are dealt round-robin to the workgroups (one per CU), and a block's
// K is walked in items of 2048 values (1 KB per row).  An item's 16 weight
// rows, 16 activation rows (rows past M read zeros) and the scales of its
// groups land in one of four LDS buffers, three items ahead (~50 KB of
// weights in flight per CU).  The only waits on these copies are the
// explicit ones at the per-item barrier; every LDS access in the loop is
// written so that the compiler adds none of its own (it cannot always tell
// the buffers apart and would wait for copies that are meant to stay in
// flight).  Each of the 8 waves multiplies 256 K values of the item: 4
// K-steps of v_mfma_i32_16x16x64_i8, two per group of 128, so every step sums
// one group.  The partial sums of the waves are added in a fixed order
// through LDS when a block ends.
//
// LDS layout of a row piece: the 64 16-byte chunks of row r (0..15) sit at
// slot (chunk ^ r), so that the 16 rows' fragment reads of one chunk hit 16
// different bank groups; the direct loads implement the swizzle by having
// lane l fetch chunk (l ^ r) (the piece stays 1 KB contiguous in memory).
//
// K order inside a wave's 256 values (bytes [128w, 128w + 128) of the piece):
// lane (row i, block kb) feeds steps 0 and 1 with chunk 8w + kb (group 2w)
// and steps 2 and 3 with chunk 8w + 4 + kb (group 2w + 1), both operands
// alike.  Widening as elsewhere: (w << 4) & 0xF0F0F0F0 and w & 0xF0F0F0F0
// give the int8 values 16*c, the MFMA returns 256*P exactly, and the 2^-8
// is applied to the finished sums (exactly: a power of two).
#include "internal.h"

namespace apex4 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int ROWS = 16;                 // weight rows per block, activation rows
constexpr int IK = 2048;                 // K values per item
constexpr int PIECE = IK / 2;            // 1024 packed bytes per row and item
constexpr int WAVES = 8;
constexpr int THREADS = WAVES * 64;
constexpr uint32_t OOB = 0x80000000u;    // past every buffer: reads zeros

struct StreamArgs {
    const uint8_t* qa;
    const float* sa;
    const uint8_t* qw;
    const float* sw;
    int M, N, K;
    int Ga, Gw;        // scale columns per row: K/ga, K/gw
    int G;             // K / gs
    int blocks;        // ceil(N / 16)
    int items;         // K items per block: ceil(K / 2048)
    _Float16* y16;
    float* y32;
    int32_t* psum;
    PsumRows prows;
};

// One item in LDS: 16 weight-row pieces, ACT activation-row pieces (ACT = 4,
// 8 or 16 >= M; the fragments of rows i >= ACT read row i mod ACT, whose
// outputs are never stored), and the scales of the item's groups: s_w as
// [16 rows][16 groups], then s_a as [16 groups][16 rows] (groups past the
// item's, rows past M: zeros; one group over K or per-channel weight scales:
// group 0 only).  RES: the ACT activation rows are instead copied to LDS
// once, whole ([row][item] pieces after the buffers), when they fit; every
// load an item needs beyond its weights costs streaming rate.  Without RES,
// the fewer activation rows an item holds, the more buffers fit.
constexpr int SC_BYTES = 2 * ROWS * 16 * 4;
template <int ACT, bool RES>
struct Item {
    static constexpr int A = ROWS * PIECE;                     // activation pieces (not RES)
    static constexpr int SC = RES ? A : A + ACT * PIECE;       // scales
    static constexpr int BYTES = SC + SC_BYTES;
    static constexpr int NBUF = RES || ACT == 16 ? 4 : ACT == 8 ? 5 : 6;  // buffers
    static constexpr int RES_A = NBUF * BYTES;                 // resident activation rows (RES)
    static constexpr int VM = RES ? 3 : 2 + (ACT == 16 ? 2 : 1) + 1;  // vector memory operations per wave and item
};
constexpr int ITEM_LDS = 144 * 1024;
static_assert(Item<16, false>::RES_A <= ITEM_LDS && Item<8, false>::RES_A <= ITEM_LDS &&
                  Item<4, false>::RES_A <= ITEM_LDS, "item buffers");
constexpr int RES_MAX = ITEM_LDS - Item<16, true>::RES_A;     // bytes of resident activation rows
__shared__ __attribute__((aligned(16))) uint8_t lds_items[ITEM_LDS];
// the waves' partial tiles of a block, two blocks apart (a block of a single
// item is finished after the next barrier while the next block is written)
__shared__ __attribute__((aligned(16))) float lds_red[2][WAVES * 64 * 4];

__device__ inline __amdgpu_buffer_rsrc_t buffer_of(const void* p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

__device__ inline uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(const lds_void*)p; }

typedef float v4f __attribute__((ext_vector_type(4)));

// LDS reads hidden from the compiler's wait analysis, each block with its own
// wait: that analysis cannot always tell the item buffers' direct-to-LDS
// copies apart, and then holds a read until copies into other buffers, in
// flight by design, have landed.  (Only the barrier orders these reads after
// the copies they need; the barrier's explicit wait covers those.)
//
// The item's operand fragments, s_a of two groups (four rows each) and s_w
// of two groups.
__device__ inline void lds_read_item(uint32_t w0a, uint32_t w1a, uint32_t x0a, uint32_t x1a, uint32_t saa,
                                     uint32_t sab, uint32_t swa, uint32_t swb, uint4& w0, uint4& w1, uint4& x0,
                                     uint4& x1, v4f& sa0, v4f& sa1, float& sw0, float& sw1)
{
    v4i r0, r1, r2, r3;
    asm volatile("ds_read_b128 %0, %8\n\t"
                 "ds_read_b128 %1, %9\n\t"
                 "ds_read_b128 %2, %10\n\t"
                 "ds_read_b128 %3, %11\n\t"
                 "ds_read_b128 %4, %12\n\t"
                 "ds_read_b128 %5, %13\n\t"
                 "ds_read_b32 %6, %14\n\t"
                 "ds_read_b32 %7, %15\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(sa0), "=&v"(sa1), "=&v"(sw0), "=&v"(sw1)
                 : "v"(w0a), "v"(w1a), "v"(x0a), "v"(x1a), "v"(saa), "v"(sab), "v"(swa), "v"(swb)
                 : "memory");
    w0 = __builtin_bit_cast(uint4, r0);
    w1 = __builtin_bit_cast(uint4, r1);
    x0 = __builtin_bit_cast(uint4, r2);
    x1 = __builtin_bit_cast(uint4, r3);
}

// the fragments only (one group over K)
__device__ inline void lds_read_frag(uint32_t w0a, uint32_t w1a, uint32_t x0a, uint32_t x1a, uint4& w0, uint4& w1,
                                     uint4& x0, uint4& x1)
{
    v4i r0, r1, r2, r3;
    asm volatile("ds_read_b128 %0, %4\n\t"
                 "ds_read_b128 %1, %5\n\t"
                 "ds_read_b128 %2, %6\n\t"
                 "ds_read_b128 %3, %7\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
                 : "v"(w0a), "v"(w1a), "v"(x0a), "v"(x1a)
                 : "memory");
    w0 = __builtin_bit_cast(uint4, r0);
    w1 = __builtin_bit_cast(uint4, r1);
    x0 = __builtin_bit_cast(uint4, r2);
    x1 = __builtin_bit_cast(uint4, r3);
}

// the 8 waves' partial values of one tile element (1 KB apart)
__device__ inline void lds_read_red(uint32_t ra, float (&v)[WAVES])
{
    asm volatile("ds_read_b32 %0, %8\n\t"
                 "ds_read_b32 %1, %8 offset:1024\n\t"
                 "ds_read_b32 %2, %8 offset:2048\n\t"
                 "ds_read_b32 %3, %8 offset:3072\n\t"
                 "ds_read_b32 %4, %8 offset:4096\n\t"
                 "ds_read_b32 %5, %8 offset:5120\n\t"
                 "ds_read_b32 %6, %8 offset:6144\n\t"
                 "ds_read_b32 %7, %8 offset:7168\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]),
                   "=&v"(v[7])
                 : "v"(ra)
                 : "memory");
}

// two scalar values
__device__ inline void lds_read_2(uint32_t a0, uint32_t a1, float& s0, float& s1)
{
    asm volatile("ds_read_b32 %0, %2\n\t"
                 "ds_read_b32 %1, %3\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(s0), "=&v"(s1)
                 : "v"(a0), "v"(a1)
                 : "memory");
}

// an LDS store hidden from the wait analysis, which would hold it until every
// direct-to-LDS copy in flight has landed; the next barrier waits for it
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

// GM: 1 (groups of 128), 2 (groups of 256), 0 (one group over K).  MIXED:
// per-channel weight scales, activation groups of 128.  ACT: activation rows
// held (M <= ACT); RES: held whole, not per item.
template <int GM, bool MIXED, bool DEBUG_P, int ACT, bool RES>
__global__ __launch_bounds__(THREADS) void gemm_stream_kernel(StreamArgs a)
{
    using L = Item<ACT, RES>;
    constexpr int NBUF = L::NBUF;
    constexpr bool SW_PER_GROUP = GM != 0 && !MIXED;       // s_w varies along K
    constexpr bool SA_PER_GROUP = GM != 0;                 // s_a varies along K
    constexpr int GPI = GM == 2 ? IK / 256 : IK / 128;     // groups per item (GM 1, 2)
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t rowbytes = (uint32_t)a.K / 2;
    const int my_blocks = blockIdx.x < a.blocks ? (a.blocks - 1 - blockIdx.x) / gridDim.x + 1 : 0;
    const int total = my_blocks * a.items;              // items of this workgroup
    const __amdgpu_buffer_rsrc_t rW = buffer_of(a.qw, (uint32_t)a.N * rowbytes);
    const __amdgpu_buffer_rsrc_t rA = buffer_of(a.qa, (uint32_t)a.M * rowbytes);
    const __amdgpu_buffer_rsrc_t rS = buffer_of(a.sw, (uint32_t)a.N * a.Gw * 4);
    const __amdgpu_buffer_rsrc_t rSA = buffer_of(a.sa, (uint32_t)a.M * a.Ga * 4);

    // --- copy of item t into buffer bi: this wave fills weight rows 2w, 2w+1
    // and activation rows 2w, 2w+1 (ACT = 16) or w mod ACT (lane l fetches
    // chunk l ^ r of row r; a row that two waves fetch gets the same bytes
    // twice), and one quarter of the scales: waves 0-3 s_w of rows
    // 4w..4w+3, waves 4-7 s_a of the item's groups 4(w-4)..4(w-4)+3; lane l
    // brings one value ---
    auto copy_item = [&](int bi, int t) {
        uint8_t* d = lds_items + bi * L::BYTES;
        float* dsc = reinterpret_cast<float*>(d + L::SC);
        const int b = blockIdx.x + gridDim.x * (t / a.items), it = t % a.items;
        const bool live = t < total;
#pragma unroll
        for (int j = 0; j < (RES ? 2 : ACT == 16 ? 4 : 3); ++j) {
            const bool act = j >= 2;
            const int r = act && ACT < 16 ? wave % ACT : 2 * wave + (j & 1);
            const uint32_t pos = (uint32_t)it * PIECE + 16 * (lane ^ r);   // byte within the row
            const uint32_t row = act ? (uint32_t)r : (uint32_t)(b * ROWS + r);
            const bool in = live && pos < rowbytes && (!act || r < a.M);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(act ? rA : rW, (lds_void*)(d + (act ? L::A : 0) + r * PIECE), 16,
                                                     in ? (int)(row * rowbytes + pos) : (int)OOB, 0, 0, 0);
        }
        if (wave < 4) {
            const int n = b * ROWS + 4 * wave + (lane >> 4), gi = lane & 15;
            const int g = SW_PER_GROUP ? it * GPI + gi : 0;
            const bool in = live && n < a.N && (SW_PER_GROUP ? gi < GPI && g < a.Gw : gi == 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rS, (lds_void*)(dsc + 64 * wave), 4,
                                                     in ? (int)(((uint32_t)n * a.Gw + g) * 4) : (int)OOB, 0, 0, 0);
        } else {
            const int m = lane & 15, gi = 4 * (wave - 4) + (lane >> 4);
            const int g = SA_PER_GROUP ? it * GPI + gi : 0;
            const bool in = live && m < a.M && (SA_PER_GROUP ? gi < GPI && g < a.Ga : gi == 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rSA, (lds_void*)(dsc + 64 * wave), 4,
                                                     in ? (int)(((uint32_t)m * a.Ga + g) * 4) : (int)OOB, 0, 0, 0);
        }
    };

    // RES: the activation rows, piece p = row * items + item (lane l fetches
    // chunk l ^ row); these copies are older than every item's, so the
    // first barrier's wait covers them
    if (RES) {
        for (int p = wave; p < ACT * a.items; p += WAVES) {
            const int r = p / a.items, it = p - r * a.items;
            const uint32_t pos = (uint32_t)it * PIECE + 16 * (lane ^ r);
            const bool in = r < a.M && pos < rowbytes;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_void*)(lds_items + L::RES_A + p * PIECE), 16,
                                                     in ? (int)(r * rowbytes + pos) : (int)OOB, 0, 0, 0);
        }
    }
    // the first NBUF - 1 items in flight
#pragma unroll
    for (int i = 0; i < NBUF - 1; ++i) copy_item(i, i);

    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    v4i P[2] = {v4i{}, v4i{}};
    int opaque_zero;                                    // zero, unknown to the compiler
    asm volatile("v_mov_b32 %0, 0" : "=v"(opaque_zero));
    const int fi = lane & 15, fkb = lane >> 4;          // fragment row, K block
    const int m_out = 4 * fkb, n_lane = lane & 15;      // output rows m_out..m_out+3, column n_lane

    // Tile element of this thread when a block is finished (threads 0-255):
    // lane ln, register r of the 16x16 tile, i.e. row m, column nl.  One
    // group over K or per-channel s_w: the group-0 scales of that element,
    // read from the block's last item while its buffer is still unchanged.
    const int f_ln = tid & 63, f_r = tid >> 6;
    const int f_m = 4 * (f_ln >> 4) + f_r, f_nl = f_ln & 15;
    float s_a0 = 0.0f, s_w0 = 0.0f;

    // The partial sums of the waves for block b (its k-th block), added in a
    // fixed order; one group over K: the exact int32 sum, then the one
    // rescale.
    auto finish_block = [&](int b, int k) {
        if (tid < ROWS * ROWS) {
            const int m = f_m, n = b * ROWS + f_nl;
            float v8[WAVES];
            lds_read_red(lds_addr(&lds_red[k & 1][f_ln * 4 + f_r]), v8);
            if (m < a.M && n < a.N) {
                float v;
                if (GM == 0) {
                    int p = 0;
#pragma unroll
                    for (int w = 0; w < WAVES; ++w) p += __builtin_bit_cast(int, v8[w]);
                    const float S = s_a0 * 0.00390625f * s_w0;
                    v = S * (float)p;
                    if (DEBUG_P)
                        if (int32_t* d = psum_at(a.psum, a.prows, m, n, a.N, 1, 0)) *d = p >> 8;
                } else {
                    v = 0.0f;
#pragma unroll
                    for (int w = 0; w < WAVES; ++w) v += v8[w];
                    v *= 0.00390625f;                    // the widening's 2^8, exactly
                    if (MIXED) v *= s_w0;
                }
                asm volatile("" : "+v"(v));   // y16 is the fp16 rounding of y32
                const int64_t off = (int64_t)m * a.N + n;
                a.y16[off] = (_Float16)v;
                if (a.y32) a.y32[off] = v;
            }
        }
    };

    // Item t uses buffer t % NBUF; the loop is unrolled by NBUF so that the
    // buffer is a compile-time choice.
    int prev_block = -1, prev_k = 0;
    for (int t0 = 0; t0 < total; t0 += NBUF)
#pragma unroll
    for (int h = 0; h < NBUF; ++h) {
        const int t = t0 + h;
        if (t >= total) break;
        const uint8_t* cur = lds_items + h * L::BYTES;
        const float* csc = reinterpret_cast<const float*>(cur + L::SC);
        const int hn = (h + NBUF - 1) % NBUF;              // (t + NBUF - 1) % NBUF, also t - 1's
        // item t has landed (the operations of the NBUF - 2 later items stay
        // in flight), and every wave is done with item t-1, whose buffer the
        // copy of t + NBUF - 1 reuses
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(waitcnt(L::VM * (NBUF - 2), 0));
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        if (prev_block >= 0) {
            finish_block(prev_block, prev_k);
            prev_block = -1;
        }
        copy_item(hn, t + NBUF - 1);

        const int b = blockIdx.x + gridDim.x * (t / a.items), it = t % a.items;
        // fragments: chunks 8w + kb and 8w + 4 + kb of row fi, swizzled
        // (activations: of row fi mod ACT)
        const int fa = fi & (ACT - 1);
        const uint8_t* wrow = cur + fi * PIECE;
        const uint8_t* arow = RES ? lds_items + L::RES_A + (fa * a.items + it) * PIECE : cur + L::A + fa * PIECE;
        const int c0 = (8 * wave + fkb) ^ fi, c1 = (8 * wave + 4 + fkb) ^ fi;
        const int a0 = (8 * wave + fkb) ^ fa, a1 = (8 * wave + 4 + fkb) ^ fa;
        uint4 w0, w1, x0, x1;
        // this wave's groups of the item: 2w, 2w + 1 (groups of 128) or w
        const int gi0 = GM == 1 ? 2 * wave : wave;
        v4f sa4[2];
        float sw2[2];
        if (GM != 0)
            lds_read_item(lds_addr(wrow + 16 * c0), lds_addr(wrow + 16 * c1), lds_addr(arow + 16 * a0),
                          lds_addr(arow + 16 * a1), lds_addr(&csc[256 + gi0 * 16 + m_out]),
                          lds_addr(&csc[256 + (gi0 + 1) * 16 + m_out]), lds_addr(&csc[n_lane * 16 + gi0]),
                          lds_addr(&csc[n_lane * 16 + gi0 + 1]), w0, w1, x0, x1, sa4[0], sa4[1], sw2[0], sw2[1]);
        else
            lds_read_frag(lds_addr(wrow + 16 * c0), lds_addr(wrow + 16 * c1), lds_addr(arow + 16 * a0),
                          lds_addr(arow + 16 * a1), w0, w1, x0, x1);
        if (GM == 1) {
            P[0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(widen_lo(x0), widen_lo(w0), v4i{}, 0, 0, 0);
            P[0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(widen_hi(x0), widen_hi(w0), P[0], 0, 0, 0);
            P[1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(widen_lo(x1), widen_lo(w1), v4i{}, 0, 0, 0);
            P[1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(widen_hi(x1), widen_hi(w1), P[1], 0, 0, 0);
        } else {
            // g = 256: the wave's 256 values are one group; one group over K:
            // the sums run through all items of the block
            v4i c = (GM == 2 || it == 0) ? v4i{} : P[0];
            c = __builtin_amdgcn_mfma_i32_16x16x64_i8(widen_lo(x0), widen_lo(w0), c, 0, 0, 0);
            c = __builtin_amdgcn_mfma_i32_16x16x64_i8(widen_hi(x0), widen_hi(w0), c, 0, 0, 0);
            c = __builtin_amdgcn_mfma_i32_16x16x64_i8(widen_lo(x1), widen_lo(w1), c, 0, 0, 0);
            P[0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(widen_hi(x1), widen_hi(w1), c, 0, 0, 0);
        }
        const int n = b * ROWS + n_lane;
        if (GM != 0) {
            // rescale this wave's group(s) of the item (the activation group
            // is the same: g_a = g, or 128 with per-channel weight scales);
            // groups past K add zero products times zero scales
            const int ng = GM == 1 ? 2 : 1;
#pragma unroll
            for (int q = 0; q < ng; ++q) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float S = MIXED ? sa4[q][r] : sa4[q][r] * sw2[q];
                    acc[r] = fmaf(S, (float)P[q][r], acc[r]);
                }
                if (DEBUG_P) {
                    const int j = it * GPI + gi0 + q;
                    if (j < a.G) {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (m_out + r < a.M && n < a.N)
                                if (int32_t* d = psum_at(a.psum, a.prows, m_out + r, n, a.N, a.G, j))
                                    *d = P[q][r] >> 8;
                    }
                }
            }
        }
        if (it == a.items - 1) {
            // the block's last item: the waves' partial sums go to LDS and are
            // added after the next barrier (one group over K: int32 sums)
            const int k = t / a.items;
            const uint32_t red = lds_addr(&lds_red[k & 1][(wave * 64 + lane) * 4]);
            if (GM == 0) {
                // (the xor is an ordinary vector instruction reading the MFMA
                // result, so the compiler puts the MFMA's result latency
                // before it; it does not for the inline-asm store)
                const v4i pv = P[0] ^ opaque_zero;
                lds_write16(red, __builtin_bit_cast(v4f, pv));
            } else {
                lds_write16(red, v4f{acc[0], acc[1], acc[2], acc[3]});
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] = 0.0f;
            }
            if ((GM == 0 || MIXED) && tid < ROWS * ROWS)
                lds_read_2(lds_addr(&csc[256 + f_m]), lds_addr(&csc[f_nl * 16]), s_a0, s_w0);
            prev_block = b;
            prev_k = k;
        }
    }
    __builtin_amdgcn_s_waitcnt(waitcnt(0, 0));
    __syncthreads();
    if (prev_block >= 0) finish_block(prev_block, prev_k);
}

template <int GM, bool MIXED, int ACT>
hipError_t launch_act(const StreamArgs& s, bool dbg, hipStream_t stream)
{
    const int grid = s.blocks < 256 ? s.blocks : 256;
    if ((int64_t)ACT * s.items * PIECE <= RES_MAX) {
        if (dbg) gemm_stream_kernel<GM, MIXED, true, ACT, true><<<grid, THREADS, 0, stream>>>(s);
        else gemm_stream_kernel<GM, MIXED, false, ACT, true><<<grid, THREADS, 0, stream>>>(s);
    } else {
        if (dbg) gemm_stream_kernel<GM, MIXED, true, ACT, false><<<grid, THREADS, 0, stream>>>(s);
        else gemm_stream_kernel<GM, MIXED, false, ACT, false><<<grid, THREADS, 0, stream>>>(s);
    }
    return hipGetLastError();
}

template <int GM, bool MIXED>
hipError_t launch_gm(const StreamArgs& s, bool dbg, hipStream_t stream)
{
    if (s.M <= 4) return launch_act<GM, MIXED, 4>(s, dbg, stream);
    if (s.M <= 8) return launch_act<GM, MIXED, 8>(s, dbg, stream);
    return launch_act<GM, MIXED, 16>(s, dbg, stream);
}

}  // namespace

bool stream_supports(const GemmProblem& p)
{
    if (p.M < 1 || p.M > ROWS || p.K % 128 != 0) return false;
    const int gs = p.ga < p.gw ? p.ga : p.gw;
    const bool mixed = p.gw == p.K && p.ga != p.gw;
    if (mixed) {
        if (p.ga != 128) return false;
    } else if (p.ga != p.gw || !(gs == 128 || gs == 256 || gs == p.K)) {
        return false;
    }
    // 32-bit buffer offsets
    const uint64_t wbytes = (uint64_t)p.N * (p.K / 2), sbytes = (uint64_t)p.N * (p.K / p.gw) * 4;
    return wbytes < OOB && sbytes < OOB && (uint64_t)p.M * (p.K / p.ga) * 4 < OOB;
}

hipError_t launch_gemm_stream(const GemmProblem& p, hipStream_t stream)
{
    StreamArgs s;
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
    const bool mixed = p.gw == p.K && p.ga != p.gw;
    const bool dbg = p.psum != nullptr;
    if (mixed) return launch_gm<1, true>(s, dbg, stream);
    if (gs == p.K && gs != 128) return launch_gm<0, false>(s, dbg, stream);   // (K = 128: one group of 128)
    if (gs == 256) return launch_gm<2, false>(s, dbg, stream);
    return launch_gm<1, false>(s, dbg, stream);
}

}  // namespace apex4
