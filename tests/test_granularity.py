"""apex4_select_granularity (include/apex4.h), a host function: the finest group
mode whose modelled speed is within the asked fraction of the fastest mode's.
The expected choices below follow from the documented model and rates by
hand (no GPU needed)."""
import pytest

from w4a4_group_quantized_amd import apex4


@pytest.fixture(scope="module", autouse=True)
def built():
    import os
    if not os.path.exists(apex4.LIB_PATH):
        pytest.skip("libapex4.so not built (run __graft_entry__.build())")


def test_prefill_picks_g128_at_65_percent():
    # compute-bound: 1565/2316 = 0.676 >= 0.65 > 834/2316 = 0.36
    assert apex4.select_granularity(2048, 12288, 4096, 0.65) == (128, 128)


def test_prefill_tighter_budgets_coarsen():
    # mixed 1672/2316 = 0.722 qualifies at 0.70 (g=128, 0.676, does not);
    # at 0.75 only g=256 (1750/2316 = 0.756) and coarser do; at 0.8 only g=K
    assert apex4.select_granularity(8192, 28672, 8192, 0.70) == (128, 8192)
    assert apex4.select_granularity(8192, 28672, 8192, 0.75) == (256, 256)
    assert apex4.select_granularity(8192, 28672, 8192, 0.80) == (8192, 8192)
    assert apex4.select_granularity(8192, 28672, 8192, 1.0) == (8192, 8192)


def test_decode_affords_fine_groups():
    # memory-bound: g=32 costs only its scale bytes, 1/(1 + 8/32) = 0.8 of g=K
    assert apex4.select_granularity(1, 28672, 8192, 0.75) == (32, 32)
    # g=64: 1/(1 + 8/64) = 0.89; g=32 (0.8) fails at 0.85
    assert apex4.select_granularity(1, 28672, 8192, 0.85) == (64, 64)


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
