// Granularity selection (include/apex4.h, apex4_select_granularity): the APEX4
// page's granularity adaptation (aiqbench news page, Abstract) for this GPU.
// The page picks the group size by how a GPU's matrix throughput compares with
// its vector throughput: where the matrix units are much faster, fine groups
// make the per-group rescale on the vector units the bottleneck.  Here that
// balance enters as the measured GEMM rate of each mode on MI355X (the
// granularity sweep M=8192, K=8192, N=28672 of bench.py), and the HBM rate
// bounds the memory-bound (decode) shapes, where fine groups cost only their
// extra scale bytes.  Host code only.
#include "apex4.h"

#include <cstdint>

namespace {

struct Mode {
    int32_t ga;        // activation group (0: K)
    int32_t gw;        // weight group (0: K)
    double ops_per_s;  // measured GEMM rate of the mode on compute-bound shapes
};

// Finest to coarsest: activation groups first (the activations carry the
// outliers), then weight groups.  Rates: bench.py --workload sweep-*, GEMM
// alone (roofline.achieved), Student-t activations, all six on one GPU
// (g = 32, 64 and 256 re-measured after kernel changes; g = 256 scaled to
// that GPU by the g = 128 rate measured beside it).
constexpr Mode kModes[] = {
    {32, 32, 581e12},
    {64, 64, 834e12},
    {128, 128, 1565e12},
    {128, 0, 1672e12},    // mixed: per-channel weights, activation groups of 128
    {256, 256, 1750e12},
    {0, 0, 2316e12},      // per-channel on both operands
};

// the weight-streaming rate the decode kernels reach (4.2-5.4 TB/s measured)
constexpr double kHbmBytesPerS = 5.0e12;

double model_seconds(const Mode& m, double M, double N, double K)
{
    const double ga = m.ga ? m.ga : K, gw = m.gw ? m.gw : K;
    const double bytes = M * K / 2 + N * K / 2 + 4 * (M * K / ga + N * K / gw) + 2 * M * N;
    const double t_mem = bytes / kHbmBytesPerS, t_ops = 2 * M * N * K / m.ops_per_s;
    return t_mem > t_ops ? t_mem : t_ops;
}

bool fits(const Mode& m, int64_t K)
{
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
        const double t = model_seconds(m, (double)M, (double)N, (double)K);
        if (best == 0.0 || t < best) best = t;
    }
    for (const Mode& m : kModes) {
        if (!fits(m, K)) continue;
        // relative speed against the fastest mode (with a hair of slack so
        // that the fastest mode always qualifies at min_rel_speed = 1)
        if (best / model_seconds(m, (double)M, (double)N, (double)K) >= min_rel_speed * (1.0 - 1e-12)) {
            *group_a = m.ga ? m.ga : (int32_t)K;
            *group_w = m.gw ? m.gw : (int32_t)K;
            return APEX4_OK;
        }
    }
    return APEX4_ERR_UNSUPPORTED;   // not reached: the fastest mode qualifies
}
