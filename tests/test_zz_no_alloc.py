"""apex4_gemm_w4a4_noalloc: the GEMM with the K splits' partial results in the
library's own per-GPU scratch array instead of a caller workspace, for callers
that cannot allocate.  Its output must equal apex4_gemm_w4a4's (same kernels,
same split, same fixed-order reduction: the same bits), on two calls in a row,
the second smaller (the array keeps the first call's contents).  Called
through the C ABI directly (ctypes), as a caller without torch would."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from w4a4_group_quantized_amd import apex4, inputs  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    apex4.lib()
    return torch.device("cuda:0")


def _noalloc(qa, sa, ga, qw, sw, gw, M, N, K, y16, y32):
    f = apex4.lib().apex4_gemm_w4a4_noalloc
    return f(apex4._ptr(qa), apex4._ptr(sa), ga, apex4._ptr(qw), apex4._ptr(sw), gw, M, N, K,
             apex4._ptr(y16), apex4._ptr(y32), torch.cuda.current_stream().cuda_stream)


def _operands(dev, M, N, K, ga, gw, seed):
    x, w = inputs.problem(M, N, K, seed=seed, act="outlier")
    qa, sa = apex4.quantize_act(torch.from_numpy(x).to(dev), ga)
    qw, sw = apex4.pack_weight(torch.from_numpy(w).to(dev), gw)
    return qa, sa, qw, sw


# (first, second): each pair takes a K split (ping-pong partial last round,
# K-outer halves) whose partial results go to the scratch array; the second
# call is smaller
PAIRS = [
    ((300, 16640, 1024, 128, 128), (130, 1000, 4096, 128, 128)),
    ((64, 8192, 8192, 128, 128), (17, 8192, 4096, 128, 128)),
    ((300, 16640, 1024, 128, 1024), (65, 640, 2048, 128, 2048)),
    ((300, 16640, 512, 64, 64), (257, 16512, 1152, 64, 64)),
]


@pytest.mark.parametrize("first,second", PAIRS)
def test_noalloc_matches_workspace_call(dev, first, second):
    for i, (M, N, K, ga, gw) in enumerate((first, second)):
        qa, sa, qw, sw = _operands(dev, M, N, K, ga, gw, seed=70 + i)
        need = apex4.workspace_size(M, N, K, ga, gw)
        assert 0 < need <= apex4.NOALLOC_MAX_WORKSPACE
        ref16, ref32, _ = apex4.gemm(qa, sa, ga, qw, sw, gw, K, want_y32=True)
        y16 = torch.full((M, N), 7.0, dtype=torch.float16, device=dev)
        y32 = torch.full((M, N), 7.0, dtype=torch.float32, device=dev)
        st = _noalloc(qa, sa, ga, qw, sw, gw, M, N, K, y16, y32)
        assert st == 0, apex4.STATUS_NAMES.get(st, st)
        torch.cuda.synchronize()
        assert torch.equal(y32.view(torch.int32), ref32.view(torch.int32)), (M, N, K)
        assert torch.equal(y16.view(torch.int16), ref16.view(torch.int16)), (M, N, K)


def test_noalloc_plain_shapes_and_refusals(dev):
    # a shape without a split needs no scratch; the result still matches
    M, N, K = 2048, 4096, 1024
    qa, sa, qw, sw = _operands(dev, M, N, K, 128, 128, seed=80)
    ref = apex4.gemm(qa, sa, 128, qw, sw, 128, K)
    y16 = torch.empty((M, N), dtype=torch.float16, device=dev)
    assert _noalloc(qa, sa, 128, qw, sw, 128, M, N, K, y16, None) == 0
    torch.cuda.synchronize()
    assert torch.equal(y16.view(torch.int16), ref.view(torch.int16))
    # the checks of apex4_gemm_w4a4 apply (nothing launched)
    assert _noalloc(qa, sa, 128, qw, sw, 128, M, N, 1000, y16, None) == 1      # K % 128
    assert _noalloc(qa, sa, 96, qw, sw, 96, M, N, K, y16, None) == 1
    # every split of this GPU fits the array: the ping-pong split takes at
    # most one 256x128 fp32 tile per compute unit
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert cus * 256 * 128 * 4 <= apex4.NOALLOC_MAX_WORKSPACE
