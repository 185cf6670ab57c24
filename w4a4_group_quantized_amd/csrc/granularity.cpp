// Granularity selection (include/apex4.h, apex4_select_granularity): the APEX4
// page's granularity adaptation (aiqbench news page, Abstract) for this GPU.
// The page picks the group size by how a GPU's matrix throughput compares with
// its vector throughput: where the matrix units are much faster, fine groups
// make the per-group rescale on the vector units the bottleneck.  Here that
// balance enters as the measured GEMM rates of each mode on MI355X, per shape
// class, for the kernel the library actually runs on the shape (the same
// choice as apex4_gemm_w4a4's): the tiled kernels of compute-bound shapes
// work in whole 256-row tiles, the weight-streaming kernels of decode shapes
// (up to 64 rows, groups of at least 128) are bound by the bytes they read.
// Groups of 32 and 64 have no streaming kernel, so at decode sizes they run
// a tiled kernel on mostly empty tiles, five times slower or more.
// Host code only.
#include "apex4.h"

#include <cmath>
#include <cstdint>

#include "internal.h"

namespace {

// Measured on MI355X (bench.py --modes, GEMM alone, back-to-back launches):
// tiled-kernel TOPS at M = 256, 2048, 4096, 8192 (the mean over the LLaMA-2
// shapes measured at that M: N = 28672 at K = 8192 for 256 and 8192; the
// 7B QKV and gate+up at 2048; the 70B QKV and gate+up at 4096), and the
// streaming kernels' algorithmic TB/s at M = 1, 4, 16, 64 (the 70B up and
// down projections; M = 4 the up projection only).
struct Mode {
    int32_t ga;        // activation group (0: K)
    int32_t gw;        // weight group (0: K)
    double tops[4];    // tiled kernels, M = 256, 2048, 4096, 8192
    double tbps[4];    // streaming kernels, M = 1, 4, 16, 64
};

// finest first: activation groups first (the activations carry the outliers),
// then weight groups
constexpr Mode kModes[] = {
    {32, 32, {538, 580, 674, 684}, {0, 0, 0, 0}},
    {64, 64, {1017, 1049, 1195, 1208}, {0, 0, 0, 0}},
    {128, 128, {1363, 1453, 1621, 1625}, {5.28, 4.33, 4.27, 2.03}},
    {128, 0, {1357, 1413, 1696, 1689}, {5.24, 4.29, 4.14, 1.99}},   // mixed: per-channel weights
    {256, 256, {1485, 1621, 1759, 1761}, {5.27, 4.33, 4.22, 1.86}},
    {0, 0, {1863, 1975, 2302, 2358}, {5.20, 4.42, 4.49, 2.30}},     // per-channel on both operands
};

constexpr double kHbmBytesPerS = 5.0e12;   // what the tiled kernels' operand reads can reach

// piecewise-linear interpolation in log2 of x over the points xs (clamped)
double interp_log2(double x, const double (&xs)[4], const double (&ys)[4])
{
    const double lx = std::log2(x);
    if (lx <= std::log2(xs[0])) return ys[0];
    for (int i = 1; i < 4; ++i) {
        const double l0 = std::log2(xs[i - 1]), l1 = std::log2(xs[i]);
        if (lx <= l1) return ys[i - 1] + (ys[i] - ys[i - 1]) * (lx - l0) / (l1 - l0);
    }
    return ys[3];
}

double model_seconds(const Mode& m, int64_t M, int64_t N, int64_t K)
{
    const int32_t ga = m.ga ? m.ga : (int32_t)K, gw = m.gw ? m.gw : (int32_t)K;
    const double Md = (double)M, Nd = (double)N, Kd = (double)K;
    const double bytes = Md * Kd / 2 + Nd * Kd / 2 + 4 * (Md * Kd / ga + Nd * Kd / gw) + 2 * Md * Nd;
    apex4::GemmProblem p{};
    p.M = (int32_t)M;
    p.N = (int32_t)N;
    p.K = (int32_t)K;
    p.ga = ga;
    p.gw = gw;
    const apex4::GemmKernel k = apex4::gemm_kernel(p);
    if (k != apex4::GemmKernel::Pingpong && k != apex4::GemmKernel::Tiled) {
        static constexpr double rows[4] = {1, 4, 16, 64};
        return bytes / (interp_log2(Md, rows, m.tbps) * 1e12);
    }
    // whole 256-row tiles of work
    static constexpr double rows[4] = {256, 2048, 4096, 8192};
    const double m_tiles = std::ceil(Md / 256.0) * 256.0;
    const double t_ops = 2 * m_tiles * Nd * Kd / (interp_log2(m_tiles, rows, m.tops) * 1e12);
    const double t_mem = bytes / kHbmBytesPerS;
    return t_mem > t_ops ? t_mem : t_ops;
}

bool fits(const Mode& m, int64_t K)
{
    if (m.ga == 0 && m.gw == 0 && K >= (int64_t(1) << 17)) return false;   // one int32 group sum over K
    return (m.ga == 0 || K % m.ga == 0) && (m.gw == 0 || K % m.gw == 0);
}

}  // namespace

extern "C" apex4_status apex4_select_granularity(int64_t M, int64_t N, int64_t K, double min_rel_speed,
                                                 int32_t* group_a, int32_t* group_w)
{
    constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;
    if (M < 1 || N < 1 || K < 128 || M > kMaxDim || N > kMaxDim || K > kMaxDim || K % 128 != 0)
        return APEX4_ERR_INVALID_ARG;
    if (!(min_rel_speed > 0.0 && min_rel_speed <= 1.0) || !group_a || !group_w) return APEX4_ERR_INVALID_ARG;
    double best = 0.0;
    for (const Mode& m : kModes) {
        if (!fits(m, K)) continue;
        const double t = model_seconds(m, M, N, K);
        if (best == 0.0 || t < best) best = t;
    }
    for (const Mode& m : kModes) {
        if (!fits(m, K)) continue;
        // relative speed against the fastest mode (with a hair of slack so
        // that the fastest mode always qualifies at min_rel_speed = 1)
        if (best / model_seconds(m, M, N, K) >= min_rel_speed * (1.0 - 1e-12)) {
            *group_a = m.ga ? m.ga : (int32_t)K;
            *group_w = m.gw ? m.gw : (int32_t)K;
            return APEX4_OK;
        }
    }
    return APEX4_ERR_UNSUPPORTED;   // not reached: the fastest mode qualifies
}
