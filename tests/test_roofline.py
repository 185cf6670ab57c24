"""Pins the roofline helper to the worked numbers printed on the blog page
"Why INT4 Weight-Only Quantization Doesn't Speed Up Prefill" (code block on where a
weight-stationary GEMM stops being memory-bound, and its printed output)."""
import pytest

from w4a4_group_quantized_amd import roofline as rl

# (peak FLOP/s, HBM B/s) as the page's table gives them
H100 = (990e12, 3.35e12)
A100 = (312e12, 2.039e12)


@pytest.mark.parametrize("spec,b,printed", [
    (H100, 2, 296), (H100, 1, 148), (H100, 0.5, 74),
    (A100, 2, 153), (A100, 0.5, 38),
])
def test_crossover_matches_printed_table(spec, b, printed):
    assert round(rl.crossover(*spec, b)) == printed


def test_mi355x_w4a4_crossover_and_bytes():
    # ridge 625 ops/B; the page's model with b = 0.5 puts the crossover at ~156 tokens
    assert rl.PEAK_INT8_OPS / rl.PEAK_HBM_BYTES == 625
    assert round(rl.crossover(rl.PEAK_INT8_OPS, rl.PEAK_HBM_BYTES, 0.5)) == 156
    # 70B up-proj decode: ~117.4 MB of packed weights + 7.34 MB of scales
    by = rl.gemm_bytes(1, 28672, 8192, 128, 128)
    assert abs(by - (28672 * 8192 / 2 + 4 * 28672 * 64 + 8192 / 2 + 4 * 64 + 2 * 28672)) < 1
    assert rl.bound_of(16, 28672, 8192, 128, 128) == "hbm"
    assert rl.bound_of(2048, 12288, 4096, 128, 128) == "mfma"
