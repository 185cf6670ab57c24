"""apex4_select_granularity (include/apex4.h), a host function: the finest group
mode whose modelled speed is within the asked fraction of the fastest mode's.
The expected choices below follow from the documented model and measured
rates by hand (no GPU needed); tests/test_gpu_granularity.py checks the
choices against GEMM times measured on the GPU."""
import pytest

from w4a4_group_quantized_amd import apex4


@pytest.fixture(scope="module", autouse=True)
def built():
    import os
    if not os.path.exists(apex4.LIB_PATH):
        pytest.skip("libapex4.so not built (run __graft_entry__.build())")


def test_prefill_picks_g128_at_65_percent():
    # compute-bound, M = 2048: 1453/1975 = 0.736 >= 0.65 > 1049/1975 = 0.531 (g=64)
    assert apex4.select_granularity(2048, 12288, 4096, 0.65) == (128, 128)


def test_prefill_picks_g64_at_half_speed():
    # groups of 64 on the ping-pong kernel: 1049/1975 = 0.531 (M = 2048) and
    # 1208/2358 = 0.512 (M = 8192) qualify at 0.5, g=32 (580/1975 = 0.294,
    # 684/2358 = 0.290) does not
    assert apex4.select_granularity(2048, 12288, 4096, 0.5) == (64, 64)
    assert apex4.select_granularity(8192, 28672, 8192, 0.5) == (64, 64)
    assert apex4.select_granularity(8192, 28672, 8192, 0.55) == (128, 128)
    assert apex4.select_granularity(8192, 28672, 8192, 0.2) == (32, 32)


def test_prefill_tighter_budgets_coarsen():
    # M = 8192: g=128 1625/2358 = 0.689 qualifies at 0.68; at 0.70 and 0.71
    # mixed (1689/2358 = 0.716) is the finest that does; at 0.72 and 0.74
    # only g=256 (1761/2358 = 0.747) and coarser; from 0.75 only g=K
    assert apex4.select_granularity(8192, 28672, 8192, 0.68) == (128, 128)
    assert apex4.select_granularity(8192, 28672, 8192, 0.70) == (128, 8192)
    assert apex4.select_granularity(8192, 28672, 8192, 0.71) == (128, 8192)
    assert apex4.select_granularity(8192, 28672, 8192, 0.72) == (256, 256)
    assert apex4.select_granularity(8192, 28672, 8192, 0.74) == (256, 256)
    assert apex4.select_granularity(8192, 28672, 8192, 0.75) == (8192, 8192)
    assert apex4.select_granularity(8192, 28672, 8192, 0.77) == (8192, 8192)
    assert apex4.select_granularity(8192, 28672, 8192, 0.80) == (8192, 8192)
    assert apex4.select_granularity(8192, 28672, 8192, 1.0) == (8192, 8192)


def test_decode_picks_a_streaming_mode():
    # M = 1, N = 28672, K = 8192: the streaming kernels read ~118-125 MB at
    # ~5.2 TB/s (mixed mode fastest, 22.4 us; g=128 23.6 us, 0.95 of it); g=32
    # and g=64 run on 256-row tiles (~225 and ~118 us)
    assert apex4.select_granularity(1, 28672, 8192, 0.75) == (128, 128)
    assert apex4.select_granularity(1, 28672, 8192, 0.96) == (128, 8192)
    for M in (1, 4, 16, 64):
        for r in (0.5, 0.75, 0.9):
            ga, gw = apex4.select_granularity(M, 28672, 8192, r)
            assert min(ga, gw) >= 128, (M, r, ga, gw)


def test_decode_fine_groups_only_on_a_tiny_budget():
    # accepting 10x slower than the fastest mode admits g=32 on 256-row tiles
    # (0.100); 5x slower g=64 (0.19)
    assert apex4.select_granularity(1, 28672, 8192, 0.05) == (32, 32)
    assert apex4.select_granularity(1, 28672, 8192, 0.09) == (32, 32)
    assert apex4.select_granularity(1, 28672, 8192, 0.11) == (64, 64)


def test_one_group_over_large_k_not_offered():
    # per-channel scales keep one int32 sum over K: refused from K = 2^17
    assert apex4.select_granularity(2048, 4096, 1 << 17, 1.0) != (1 << 17, 1 << 17)
    assert apex4.select_granularity(2048, 4096, (1 << 17) - 128, 1.0) == ((1 << 17) - 128, (1 << 17) - 128)


def test_modes_that_do_not_divide_k_are_skipped():
    # K = 384: g=256 does not divide it; at 0.8 the compute-bound choice is mixed
    ga, gw = apex4.select_granularity(8192, 8192, 384, 0.8)
    assert 384 % ga == 0 and 384 % gw == 0


def test_monotone_in_the_budget():
    order = [(32, 32), (64, 64), (128, 128), (128, 4096), (256, 256), (4096, 4096)]
    for M in (1, 16, 64, 256, 2048):
        prev = -1
        for r in (0.3, 0.5, 0.7, 0.8, 0.9, 0.95, 1.0):
            i = order.index(apex4.select_granularity(M, 8192, 4096, r))
            assert i >= prev
            prev = i


@pytest.mark.parametrize("args", [(0, 8, 128, 0.5), (8, 0, 128, 0.5), (8, 8, 64, 0.5), (8, 8, 200, 0.5),
                                  (8, 8, 128, 0.0), (8, 8, 128, 1.5)])
def test_invalid_arguments(args):
    with pytest.raises(apex4.Apex4Error):
        apex4.select_granularity(*args)
