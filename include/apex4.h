/*
 * apex4.h -- C ABI of the MI355X (gfx950) pure W4A4 group-quantized GEMM.
 *
 * The operation is the one "APEX4: Efficient Pure W4A4 LLM Inference via
 * Intra-SM Compute Rebalancing" (aiqbench news page, Abstract) builds its
 * kernels around: weights and activations both symmetric 4-bit integers with
 * one scale per row per K-group ("W4A4-g128" for groups of 128), an integer
 * matrix product per group, and a per-group rescale ("group dequantization")
 * accumulated in fp32:
 *
 *     Y[m,n] = sum_j s_a[m,j] * s_w[n,j] * sum_{k in group j} qa[m,k] * qw[n,k]
 *
 * The same page's granularity adaptation makes the group size selectable, and
 * its mixed-granularity mode is supported as per-channel weight scales
 * (group_w == K) with grouped activation scales.
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers (HIP device memory on the current device)
 *     unless a comment says otherwise.  Every tensor is row-major and
 *     contiguous.  The caller owns every buffer; the library allocates nothing,
 *     frees nothing and keeps no state between calls (beyond a host-side cache
 *     of each device's compute-unit count), so calls are re-entrant.
 *   - Packed INT4 tensors hold two's-complement 4-bit codes, two per byte, code
 *     k of a row in byte k/2, the even k in the low nibble.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Calls are
 *     asynchronous and ordered on that stream; results are ready once the
 *     stream has been synchronized.
 *   - Arguments are checked on the host before anything is launched.  A
 *     failed check returns a status code below and touches no memory.  A
 *     launch failure returns APEX4_ERR_HIP.  Faults during execution surface at
 *     the caller's next synchronization.  No C++ exception crosses this ABI.
 *   - Inputs must be finite; results for NaN or Inf inputs are unspecified.
 */
#ifndef APEX4_H
#define APEX4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t apex4_status;

#define APEX4_OK 0
#define APEX4_ERR_INVALID_ARG 1  /* a size or pointer is out of the documented range */
#define APEX4_ERR_UNSUPPORTED 2  /* a group-size combination this library does not run */
#define APEX4_ERR_ALIGNMENT 3    /* a pointer lacks the documented alignment */
#define APEX4_ERR_WORKSPACE 4    /* workspace smaller than apex4_gemm_workspace_size() */
#define APEX4_ERR_HIP 5          /* the HIP runtime reported an error at launch */

/* Static string naming a status code (host function; never NULL). */
const char* apex4_status_string(apex4_status s);

/*
 * Symmetric per-group INT4 quantization of fp16 activations, done online per
 * token (APEX4 page, Abstract: pure W4A4, activations quantized alongside the
 * weights).  For each row m and group j (k in [j*g, (j+1)*g)):
 *     a = max_k |x[m,k]|;  s_a[m,j] = a / 7 (fp32, correctly rounded);
 *     qa[m,k] = clamp(round_half_even(x[m,k] / s_a[m,j]), -8, 7)
 *               (fp32 correctly rounded quotient);  a == 0 gives s = 0, q = 0.
 *   x_f16  [M, K] fp16, 16-byte aligned.
 *   qa_u8  [M, K/2] packed codes (output), 4-byte aligned.
 *   s_a    [M, K/group_a] fp32 (output), 4-byte aligned.
 *   M >= 0 (0 is a no-op), K > 0, K % 8 == 0,
 *   group_a in {32, 64, 128, 256} or group_a == K, K % group_a == 0.
 * Output is bit-identical to the reference rule above.
 */
apex4_status apex4_quantize_act(const void* x_f16, int64_t M, int64_t K, int32_t group_a,
                                void* qa_u8, float* s_a, void* stream);

/*
 * Offline weight packing (APEX4 page, Abstract: the INT4 GEMM consumes INT4
 * weights): the same per-group rule as apex4_quantize_act, applied to the rows
 * of W [N, K] (output channels by input features), producing the canonical
 * packed layout apex4_gemm_w4a4 reads.
 *   w_f16 [N, K] fp16, 16-byte aligned; qw_u8 [N, K/2]; s_w [N, K/group_w].
 *   Same size and group rules as apex4_quantize_act (group_w == K gives the
 *   per-channel scales of the mixed-granularity mode).
 */
apex4_status apex4_pack_weight(const void* w_f16, int64_t N, int64_t K, int32_t group_w,
                               void* qw_u8, float* s_w, void* stream);

/*
 * Bytes of device workspace apex4_gemm_w4a4 needs for this shape (host
 * function; it reads the current device's compute-unit count).  Nonzero only
 * where the compute-bound kernel (groups of 128, M > 64, K >= 512) would leave
 * its last round of 256 x 128 output tiles (its only one, for few tiles) at
 * most half the GPU's compute units: those tiles then run as P = min(CUs /
 * tiles, K / 256, 4) parts of K into fp32 partial tiles in the workspace
 * (P x tiles x 256 x 128 x 4 bytes, e.g. 25.2 MB for M = 2048, N = 22016 on
 * 256 CUs) and a reduction adds the parts in a fixed order.  Also nonzero
 * for 17 <= M <= 64 rows (groups of 128 or mixed) when the 16-column blocks
 * leave at most 2 per compute unit and K > 3072: the kernel then walks two
 * halves of K (2 x M x N x 4 bytes, e.g. 4 MB for M = 64, N = 8192).  0 for
 * invalid or empty shapes.  The workspace holds nothing between calls; calls
 * that overlap on one workspace race.
 */
size_t apex4_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int32_t group_a,
                                 int32_t group_w);

/*
 * The W4A4 GEMM with per-group dequantization (APEX4 page, Abstract: INT4
 * products summed per group, each group rescaled and accumulated on the
 * vector units), Y = X * W^T in the quantized domain:
 *     P_j[m,n] = sum_{k in group j} qa[m,k] * qw[n,k]          (exact int32)
 *     Y[m,n]   = sum_j s_a[m, j*gs/group_a] * s_w[n, j*gs/group_w] * P_j[m,n]
 * with gs = min(group_a, group_w) and G = K/gs groups, accumulated in fp32.
 * The fp32 summation order is not fixed (the result is within 1e-5 of
 * max|Y| of the ascending-order sum); P_j is exact.
 *   qa_u8  [M, K/2] packed, 16-byte aligned;  s_a [M, K/group_a] fp32.
 *   qw_u8  [N, K/2] packed, 16-byte aligned;  s_w [N, K/group_w] fp32.
 *   y_f16  [M, N] fp16 output (round to nearest even), 2-byte aligned.
 *   y_f32  [M, N] fp32 output before the fp16 rounding, or NULL.
 *   psum_dbg [M, N, G] int32 per-group sums P_j, or NULL (debug; slow).
 *   workspace / workspace_bytes: at least apex4_gemm_workspace_size() bytes
 *   (NULL allowed when that is 0), 16-byte aligned; device memory owned by the
 *   caller, overwritten by the call.
 * Sizes: M >= 0, N >= 0 (either 0 is a no-op), K > 0, K % 128 == 0,
 *   group_a in {32, 64, 128, 256} or group_a == K, and either
 *   group_w == group_a, or group_w == K (mixed granularity: per-channel
 *   weights, grouped activations).  M, N, K < 2^31 and M*N*G < 2^31 when
 *   psum_dbg is given.  One group over all of K (group_a == group_w == K)
 *   needs K < 2^17 = 131072: the group's integer sum is held in one int32
 *   register as 256 times its value (the codes enter the int8 matrix
 *   instruction as 16 c), and 256 * 64 * K must stay below 2^31.  Larger K
 *   with one group returns APEX4_ERR_UNSUPPORTED (groups of at most 256, or
 *   mixed mode, have no such limit).
 */
apex4_status apex4_gemm_w4a4(const void* qa_u8, const float* s_a, int32_t group_a,
                             const void* qw_u8, const float* s_w, int32_t group_w,
                             int64_t M, int64_t N, int64_t K,
                             void* y_f16, float* y_f32, int32_t* psum_dbg,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * apex4_gemm_w4a4 with the per-group sums of selected rows only, for checking
 * large shapes in the launch configuration apex4_gemm_w4a4 uses (debug; slow).
 * Output row m = p_row0 + i * p_step (i < p_rows) has its sums P_j[m, n] in
 * psum_dbg[i, n, j] (int32 [p_rows, N, G]); no other row's sums are written.
 * Y, y_f32 and every other argument are exactly those of apex4_gemm_w4a4,
 * whose psum_dbg is this call with p_row0 = 0, p_step = 1, p_rows = M.
 *   p_row0 >= 0, p_step >= 1, p_rows >= 0 (0: no sums, psum_dbg may be NULL),
 *   p_row0 + (p_rows - 1) * p_step < M, p_rows * N * G < 2^31;
 *   otherwise APEX4_ERR_INVALID_ARG, found on the host before any launch.
 */
apex4_status apex4_gemm_w4a4_debug(const void* qa_u8, const float* s_a, int32_t group_a,
                                   const void* qw_u8, const float* s_w, int32_t group_w,
                                   int64_t M, int64_t N, int64_t K, void* y_f16, float* y_f32,
                                   int64_t p_row0, int64_t p_step, int64_t p_rows, int32_t* psum_dbg,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * apex4_gemm_w4a4 for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * There is no workspace argument: the only scratch memory of the GEMM (the
 * fp32 partial results of its K splits, see apex4_gemm_workspace_size) goes to
 * an array the library holds in the memory of every GPU it runs on, of
 * APEX4_NOALLOC_MAX_WORKSPACE bytes, from module load until the process ends.
 * Arguments, checks, status codes and results are those of apex4_gemm_w4a4
 * without debug sums (the same kernels and the same K splits, so the same
 * bits).  A shape whose apex4_gemm_workspace_size() exceeds the array returns
 * APEX4_ERR_WORKSPACE before anything is launched (on MI355X none does: the
 * largest split takes one 256 x 128 fp32 tile per compute unit, 32 MiB on 256
 * compute units).  The call itself allocates nothing; its first call on a
 * device looks up that device's array address (hipGetSymbolAddress; a
 * failure returns APEX4_ERR_HIP).  The array keeps the last call's contents
 * and is fully rewritten before it is read; calls that overlap on one GPU
 * (concurrent streams or threads) share it and race.
 */
#define APEX4_NOALLOC_MAX_WORKSPACE ((size_t)32 << 20)
apex4_status apex4_gemm_w4a4_noalloc(const void* qa_u8, const float* s_a, int32_t group_a,
                                     const void* qw_u8, const float* s_w, int32_t group_w,
                                     int64_t M, int64_t N, int64_t K, void* y_f16, float* y_f32,
                                     void* stream);

/*
 * One W4A4 linear layer call: Y = X * W^T with X quantized on the fly, i.e.
 * apex4_quantize_act(X) followed by apex4_gemm_w4a4 (the APEX4 page,
 * Abstract: activations quantized online, weights offline), with the same
 * codes, scales and result bits as those two calls.  With 1 or 2 rows,
 * activation groups of 128 or 256 and K <= 8192 the decode kernel quantizes
 * the rows itself (one launch, no round trip of the codes through memory;
 * for larger K every workgroup's read of the fp16 rows costs more than the
 * separate launch); otherwise the quantization runs into the workspace and
 * the GEMM follows.
 *   x_f16 [M, K] fp16, 16-byte aligned; qw_u8, s_w, the groups, M, N, K, y_f16
 *   and y_f32 as in apex4_gemm_w4a4 (no debug sums).
 *   workspace / workspace_bytes: at least apex4_linear_workspace_size() bytes
 *   (0 for the fused shapes), 256-byte aligned; caller-owned, overwritten
 *   (the activation codes, then their scales, each part 256-byte aligned,
 *   then the GEMM's own workspace); calls that share one workspace race.
 *   Errors: APEX4_ERR_INVALID_ARG (shapes, groups, null pointers),
 *   APEX4_ERR_UNSUPPORTED (a group combination the quantizer or the GEMM does
 *   not run), APEX4_ERR_ALIGNMENT, APEX4_ERR_WORKSPACE, APEX4_ERR_HIP; all
 *   but the last are found on the host before anything is enqueued.  M == 0
 *   or N == 0 is a no-op.  The work is enqueued on `stream` and the call
 *   returns before it runs.  apex4_linear_workspace_size returns 0 for
 *   invalid arguments (the call then reports them).
 */
size_t apex4_linear_workspace_size(int64_t M, int64_t N, int64_t K, int32_t group_a, int32_t group_w);
apex4_status apex4_linear_w4a4(const void* x_f16, int32_t group_a, const void* qw_u8, const float* s_w,
                               int32_t group_w, int64_t M, int64_t N, int64_t K, void* y_f16, float* y_f32,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * FP8-coded operands: a variant of the same GEMM whose operands hold one byte
 * per code instead of two nibbles.  The INT4 codes -8..7 are exact values of
 * FP8 E4M3 (the OCP format of gfx950), and gfx950's FP8 matrix instruction
 * (v_mfma_scale_f32_32x32x64_f8f6f4, unit block scales) sums their exact
 * products in fp32, which for these integers is exact (|group sum| <= 64 *
 * 128 < 2^24): the per-group sums P_j and the result are those of
 * apex4_gemm_w4a4, while the int32 -> fp32 conversion of the rescale and the
 * nibble widening go away.  The price is twice the operand bytes.  (The OSC
 * page, Abstract, points to 4-bit micro-scaling matrix hardware as the way
 * ahead; the APEX4 page's own kernels run on INT4 tensor cores.)
 *
 * apex4_quantize_f8: the quantization rule of apex4_quantize_act /
 * apex4_pack_weight (groups of 64 or 128), codes written as E4M3 bytes, one
 * per element in K order (-0 is written as +0).
 *   x_f16 [rows, K] fp16, 16-byte aligned; rows >= 0 (0: no-op), K % group == 0.
 *   q8 [rows, K] bytes, 8-byte aligned;  s [rows, K/group] fp32, as apex4_quantize_act.
 *   group: 64 or 128 (other valid groups: APEX4_ERR_UNSUPPORTED).
 */
apex4_status apex4_quantize_f8(const void* x_f16, int64_t rows, int64_t K, int32_t group, void* q8,
                               float* s, void* stream);

/*
 * apex4_gemm_w4a4_f8: Y of apex4_gemm_w4a4 with group_a = group_w = group
 * from E4M3-coded operands (apex4_quantize_f8 outputs).
 *   qa8 [M, K], qw8 [N, K] bytes, 16-byte aligned; s_a [M, K/group], s_w [N, K/group].
 *   group: 64 or 128 on both operands (other divisors of K: APEX4_ERR_UNSUPPORTED).
 *   At groups of 64 the matrix instruction's fp32 result is the group sum
 *   itself, and the rescale is one fma per output and group where the INT4
 *   path also converts the int32 sum.
 *   y_f16 [M, N], y_f32 [M, N] or NULL, psum_dbg [M, N, K/group] int32 or NULL,
 *   as in apex4_gemm_w4a4 (the fp32 summation order is not fixed; P exact).
 *   M, N >= 0 (0: no-op), K > 0, K % 128 == 0, 256 * K < 2^31.  Any M works;
 *   the kernel is the compute-bound one (256 x 128 output tiles), meant for
 *   prefill-sized M.  No workspace.  Asynchronous on `stream`.
 */
apex4_status apex4_gemm_w4a4_f8(const void* qa8, const float* s_a, const void* qw8, const float* s_w,
                                int32_t group, int64_t M, int64_t N, int64_t K, void* y_f16, float* y_f32,
                                int32_t* psum_dbg, void* stream);

/*
 * FP6-coded operands: the same GEMM with each INT4 code stored as a 6-bit
 * FP6 E2M3 field, the operand format gfx950's micro-scaling matrix
 * instruction (v_mfma_scale_f32_32x32x64_f8f6f4) reads at twice its int8
 * rate (the OSC page, Abstract, looks to 4-bit micro-scaling matrix hardware;
 * the method is that of the APEX4 page, Abstract).  A code c in [-8, 7] is
 * the field (c < 0) << 5 | |c|: with exponent bias 1 and 3 mantissa bits,
 * the magnitudes 0..15 are the values 0/8 .. 15/8, so the field is c / 8
 * exactly; the instruction's E8M0 block scales (2^3 on both operands) undo
 * the 1/8, and its fp32 sum of products of such integers is exact.  The
 * group sums P_j, and hence Y, are those of apex4_gemm_w4a4 on the same codes;
 * the codes need no unpacking and the rescale no int -> fp32 conversion.  The
 * price is 6 bits per code instead of 4.
 *
 * apex4_quantize_f6: the quantization rule of apex4_quantize_act /
 * apex4_pack_weight (groups of 128), codes written as E2M3 fields (-0 is
 * written as +0).  The 128 fields of a (row, group) pack little-endian into
 * 96 bytes (code k of the group at bits 6k .. 6k+5), i.e. six 16-byte
 * chunks.  Tiled layout: rows in blocks of 64, the last block padded with
 * zero rows; the tile of row block b and group j is 6 KB at byte
 * (b * K/128 + j) * 6144, and chunk q of row i of the block sits at
 * + q * 1024 + i * 16 (each chunk of 64 rows is one contiguous KB, the piece
 * the GEMM moves from memory to LDS in one load).
 *   x_f16 [rows, K] fp16, 16-byte aligned; rows >= 0 (0: no-op), K % 128 == 0.
 *   q6: ceil(rows/64)*64 * 3K/4 bytes (padding rows written as zeros),
 *       16-byte aligned;  s [rows, K/128] fp32, as apex4_quantize_act.
 *   group: 128 only (other valid groups: APEX4_ERR_UNSUPPORTED).
 */
apex4_status apex4_quantize_f6(const void* x_f16, int64_t rows, int64_t K, int32_t group, void* q6,
                               float* s, void* stream);

/*
 * apex4_gemm_w4a4_f6: Y of apex4_gemm_w4a4 with group_a = group_w = 128 from
 * FP6-coded operands (apex4_quantize_f6 outputs, tiled layout).
 *   qa6: ceil(M/64)*64 * 3K/4 bytes, qw6: ceil(N/64)*64 * 3K/4 bytes, both
 *   16-byte aligned, padding rows zero; s_a [M, K/128], s_w [N, K/128] fp32.
 *   y_f16 [M, N], y_f32 [M, N] or NULL, psum_dbg [M, N, K/128] int32 or NULL
 *   (M*N*K/128 < 2^31), as in apex4_gemm_w4a4.
 *   workspace: at least apex4_gemm_workspace_size(M, N, K, 128, 128) bytes
 *   (the same K split of a partial last round of 256x128 tiles), 16-byte
 *   aligned, caller-owned.
 *   M, N >= 0 (0: no-op), K > 0, K % 128 == 0, 4 * 6144 * K/128 < 2^31
 *   (APEX4_ERR_UNSUPPORTED otherwise).  The kernel is the compute-bound one
 *   (256 x 128 output tiles), meant for prefill-sized M.  Asynchronous on
 *   `stream`; every check runs on the host before anything is launched.
 */
apex4_status apex4_gemm_w4a4_f6(const void* qa6, const float* s_a, const void* qw6, const float* s_w,
                                int64_t M, int64_t N, int64_t K, void* y_f16, float* y_f32,
                                int32_t* psum_dbg, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Granularity selection for a GEMM shape on this GPU (APEX4 page, Abstract:
 * granularity adaptation by the GPU's matrix-to-vector throughput balance).
 * The modes, finest first: g = 32, 64, 128; mixed (group_a = 128, group_w =
 * K); g = 256; per-channel (g = K).  Each mode's time on the shape is modelled
 * from GEMM rates measured on MI355X for the kernel apex4_gemm_w4a4 runs on
 * that shape and mode:
 *   - up to 64 rows with groups of at least 128 (the weight-streaming
 *     kernels): bytes / rate, with the algorithmic bytes
 *     M*K/2 + N*K/2 + 4*(M*K/group_a + N*K/group_w) + 2*M*N and the rate
 *     interpolated (in log2 M) from the measured TB/s at M = 1, 4, 16, 64
 *     (about 5.2, 4.3, 4.3, 2.0 TB/s);
 *   - otherwise the tiled kernels, which work in whole 256-row tiles:
 *     max(bytes / 5.0e12 B/s, 2*M'*N*K / rate) with M' = M rounded up to a
 *     multiple of 256 and the rate interpolated from the measured TOPS at
 *     M' = 256, 2048, 4096, 8192 (g = 32: 538..684, 64: 1017..1208, 128:
 *     1363..1625, mixed: 1357..1696, 256: 1485..1761, K: 1863..2358).
 * Groups of 32 and 64 have no weight-streaming kernel: at decode sizes they
 * run on mostly empty 256-row tiles and are modelled (and measured) five or
 * more times slower.  The finest mode whose modelled speed is at least
 * min_rel_speed times the fastest mode's is returned.  Modes whose groups do
 * not divide K are skipped, and so is one group over K for K >= 2^17 (see
 * apex4_gemm_w4a4).  Host function: touches no device memory.
 *   M, N >= 1; K >= 128, K % 128 == 0; 0 < min_rel_speed <= 1.
 *   group_a, group_w: HOST int32 outputs (group_w == K for per-channel
 *   weights), valid arguments for apex4_quantize_act / apex4_pack_weight /
 *   apex4_gemm_w4a4.
 */
apex4_status apex4_select_granularity(int64_t M, int64_t N, int64_t K, double min_rel_speed,
                                      int32_t* group_a, int32_t* group_w);

#ifdef __cplusplus
}
#endif

#endif /* APEX4_H */
