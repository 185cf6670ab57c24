/*
 * CPU oracle for the pure W4A4 group-quantized GEMM -- TEST INFRASTRUCTURE ONLY.
 *
 * Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may load
 * this file's library.  The product path (the HIP library) never calls it and
 * shares no code with it.
 *
 * What it computes follows "APEX4: Efficient Pure W4A4 LLM Inference via
 * Intra-SM Compute Rebalancing" (aiqbench news page, Abstract): both operands
 * are 4-bit integers ("pure W4A4"), the integer products of each K-group are
 * summed exactly (the INT4 tensor-core part) and every group's integer sum is
 * rescaled on the vector units ("group dequantization") before it is added to
 * the output.  The page gives that formula only in words; written out,
 *
 *     Y[m,n] = sum_j  s_a[m,j] * s_w[n,j] * sum_{k in group j} qa[m,k]*qw[n,k]
 *
 * with one symmetric scale per row per K-group for each operand.  The details
 * the page leaves open are taken as follows (each is a reading, listed with its
 * reason in the design notes of the repository):
 *   - quantization is symmetric, s = absmax / 7 in fp32, q = round-half-even
 *     (x / s) with an IEEE fp32 division, clamped to [-8, 7]; an all-zero group
 *     gets s = 0 and q = 0;
 *   - two's-complement nibbles, the even k in the low nibble of each byte,
 *     rows K-contiguous: packed [rows, K/2] bytes, scales [rows, K/g] fp32;
 *   - the fp32 combination is, for each group j in ascending order,
 *     S_j = s_a*s_w, t_j = S_j*float(P_j), acc = acc + t_j, with no fused
 *     multiply-add (built with -ffp-contract=off); the fp16 output is acc
 *     rounded to nearest even;
 *   - the mixed-granularity mode named on the same page is per-channel weight
 *     scales (g_w = K) with grouped activation scales; it is the same formula,
 *     since the weight scale index j*g/g_w is then 0 for every group.
 *
 * Plain C11, no blocking, no reordering beyond the definition above.  OpenMP
 * only splits the independent output rows.  Non-finite inputs are rejected.
 */
#include <math.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_ERR_ARG 1
#define ORACLE_ERR_NONFINITE 2
#define ORACLE_ERR_NOMEM 3

/* ---- IEEE binary16 <-> binary32, from the format's definition ----------- */

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
float oracle_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    float mag;
    if (e == 0)
        mag = ldexpf((float)f, -24);                /* subnormal: f * 2^-24 */
    else if (e == 31)
        mag = f ? NAN : INFINITY;
    else
        mag = ldexpf((float)(1024 + f), e - 25);    /* (1 + f/1024) * 2^(e-15) */
    return sign ? -mag : mag;
}

/* Round a binary32 value to the nearest binary16 value, ties to even. */
uint16_t oracle_f32_to_f16(float x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    float a = fabsf(x);
    if (isnan(x))
        return (uint16_t)(sign | 0x7e00);
    if (isinf(a))
        return (uint16_t)(sign | 0x7c00);
    if (a < ldexpf(1.0f, -14)) {
        /* subnormal range: the quantum is 2^-24; 1024 quanta is the smallest normal */
        float q = nearbyintf(ldexpf(a, 24));
        return (uint16_t)(sign | (uint16_t)q);
    }
    int e;
    frexpf(a, &e);          /* a = m * 2^e, m in [0.5, 1): exponent of a is e-1 */
    int ex = e - 1;
    float m = nearbyintf(ldexpf(a, 10 - ex));       /* significand in [1024, 2048] */
    if (m == 2048.0f) {
        m = 1024.0f;
        ex += 1;
    }
    if (ex > 15)
        return (uint16_t)(sign | 0x7c00);           /* rounds past 65504: inf */
    return (uint16_t)(sign | (uint16_t)((ex + 15) << 10) | (uint16_t)((int)m - 1024));
}

/* ---- symmetric per-group INT4 quantization and nibble packing ------------ */

/* Encode one code in [-8, 7] as a two's-complement nibble. */
static uint8_t nibble_of(int q) { return (uint8_t)(q & 0xf); }

/* Decode a two's-complement nibble to [-8, 7]. */
static int code_of(uint8_t nib) { return nib >= 8 ? (int)nib - 16 : (int)nib; }

/* Code k of a packed row: byte k/2, low nibble for even k. */
int oracle_code_at(const uint8_t* row, int64_t k)
{
    uint8_t b = row[k / 2];
    return code_of((k % 2 == 0) ? (uint8_t)(b & 0xf) : (uint8_t)(b >> 4));
}

/*
 * x: fp16 bit patterns [rows, K]; g divides K, K even.
 * q: packed codes [rows, K/2]; s: fp32 scales [rows, K/g].
 */
int oracle_quantize(const uint16_t* x, int64_t rows, int64_t K, int64_t g,
                    uint8_t* q, float* s)
{
    if (!x || !q || !s || rows < 0 || K <= 0 || g <= 0 || K % g != 0 || K % 2 != 0)
        return ORACLE_ERR_ARG;
    for (int64_t i = 0; i < rows * K; ++i)
        if (!isfinite(oracle_f16_to_f32(x[i])))
            return ORACLE_ERR_NONFINITE;

    const int64_t G = K / g;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t* xr = x + r * K;
        uint8_t* qr = q + r * (K / 2);
        memset(qr, 0, (size_t)(K / 2));
        for (int64_t j = 0; j < G; ++j) {
            /* step 1: the group's absolute maximum (exact in fp32) */
            float amax = 0.0f;
            for (int64_t k = j * g; k < (j + 1) * g; ++k) {
                float v = fabsf(oracle_f16_to_f32(xr[k]));
                if (v > amax)
                    amax = v;
            }
            /* step 2: the scale, one correctly rounded fp32 division */
            float sc = amax / 7.0f;
            s[r * G + j] = (amax == 0.0f) ? 0.0f : sc;
            /* step 3: codes, round half to even of an fp32 quotient, clamped */
            for (int64_t k = j * g; k < (j + 1) * g; ++k) {
                int code = 0;
                if (amax != 0.0f) {
                    float v = nearbyintf(oracle_f16_to_f32(xr[k]) / sc);
                    if (v < -8.0f) v = -8.0f;
                    if (v > 7.0f) v = 7.0f;
                    code = (int)v;
                }
                /* step 4: pack, even k in the low nibble */
                if (k % 2 == 0)
                    qr[k / 2] |= nibble_of(code);
                else
                    qr[k / 2] |= (uint8_t)(nibble_of(code) << 4);
            }
        }
    }
    return ORACLE_OK;
}

/* ---- the GEMM: exact integer group sums, fp32 rescale-accumulate --------- */

/*
 * qa: packed [M, K/2], s_a: [M, K/ga]; qw: packed [N, K/2], s_w: [N, K/gw].
 * Groups are the finer of the two partitions, gs = min(ga, gw), G = K/gs.
 * Outputs (each may be NULL): y16 fp16 bits [M, N], y32 [M, N], p int32 [M, N, G].
 */
int oracle_gemm(const uint8_t* qa, const float* s_a, int64_t ga,
                const uint8_t* qw, const float* s_w, int64_t gw,
                int64_t M, int64_t N, int64_t K,
                uint16_t* y16, float* y32, int32_t* p)
{
    if (!qa || !s_a || !qw || !s_w || M < 0 || N < 0 || K <= 0 || K % 2 != 0 ||
        ga <= 0 || gw <= 0 || K % ga != 0 || K % gw != 0)
        return ORACLE_ERR_ARG;
    const int64_t gs = ga < gw ? ga : gw;
    if (ga % gs != 0 || gw % gs != 0)
        return ORACLE_ERR_ARG;
    const int64_t G = K / gs, Ga = K / ga, Gw = K / gw;
    for (int64_t i = 0; i < M * Ga; ++i)
        if (!isfinite(s_a[i])) return ORACLE_ERR_NONFINITE;
    for (int64_t i = 0; i < N * Gw; ++i)
        if (!isfinite(s_w[i])) return ORACLE_ERR_NONFINITE;

    /* Decode both operands to one code per byte first (a plain lookup). */
    int8_t* ca = (int8_t*)malloc((size_t)(M * K) + 1);
    int8_t* cw = (int8_t*)malloc((size_t)(N * K) + 1);
    if (!ca || !cw) {
        free(ca);
        free(cw);
        return ORACLE_ERR_NOMEM;
    }
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k)
            ca[m * K + k] = (int8_t)oracle_code_at(qa + m * (K / 2), k);
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            cw[n * K + k] = (int8_t)oracle_code_at(qw + n * (K / 2), k);

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            float acc = 0.0f;
            for (int64_t j = 0; j < G; ++j) {
                /* exact integer sum over the group */
                int64_t pj = 0;
                for (int64_t k = j * gs; k < (j + 1) * gs; ++k)
                    pj += (int64_t)ca[m * K + k] * (int64_t)cw[n * K + k];
                /* fp32 rescale and accumulate, ascending j, no FMA */
                float S = s_a[m * Ga + (j * gs) / ga] * s_w[n * Gw + (j * gs) / gw];
                float t = S * (float)pj;
                acc = acc + t;
                if (p)
                    p[(m * N + n) * G + j] = (int32_t)pj;
            }
            if (y32)
                y32[m * N + n] = acc;
            if (y16)
                y16[m * N + n] = oracle_f32_to_f16(acc);
        }
    }
    free(ca);
    free(cw);
    return ORACLE_OK;
}

/* Number of OpenMP threads the oracle runs on (for the cpu baseline report). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
