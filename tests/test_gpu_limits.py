"""Sizes past 32-bit byte offsets, against the CPU oracle.

The decode kernels address their weights with 32-bit buffer offsets and
refuse packed weights of 2 GiB or more; such calls run on a tiled kernel,
which bases every workgroup's pointers in 64 bits.  The quantization kernels
index chunks in 64 bits.  These tests cross both limits at their real sizes
and check sampled outputs: the oracle computes them one by one.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import oracle as orc  # noqa: E402
from w4a4_group_quantized_amd import apex4, inputs  # noqa: E402

REL_TOL = 1e-5


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    apex4.lib()
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def big_weights(dev):
    """2 GiB of uniform random packed weight bytes (N = 131072, K = 32768)
    with random scales for groups of 64 (the 128-group scales are taken as
    every other column, so both group sizes see the same codes)."""
    N, K = 131072, 32768
    q, s = inputs.random_packed(N, K, K // 64, seed=2024)
    assert q.nbytes == 2**31
    tq = torch.from_numpy(q).to(dev)
    return N, K, q, s, tq


@pytest.mark.gpu
@pytest.mark.parametrize("M,g", [(1, 128), (40, 128), (3, 64)])
def test_gemm_weights_of_2gib(dev, big_weights, M, g):
    N, K, q, s64, tq = big_weights
    s = np.ascontiguousarray(s64[:, ::g // 64])
    ts = torch.from_numpy(s).to(dev)
    qa, sa = inputs.random_packed(M, K, K // g, seed=M)
    y16, y32, _ = apex4.gemm(torch.from_numpy(qa).to(dev), torch.from_numpy(sa).to(dev), g, tq, ts, g, K,
                             want_y32=True)
    torch.cuda.synchronize()
    cols = np.array([0, 1, 127, 128, 65535, 65536, 100000, 131070, 131071])
    _, r32, _ = orc.gemm(qa, sa, g, q[cols], s[cols], g, K)
    got = y32.cpu().numpy()[:, cols].astype(np.float64)
    tol = REL_TOL * float(np.abs(r32).max())
    assert float(np.abs(got - r32).max()) <= tol
    assert np.array_equal(y16.cpu().numpy()[:, cols].view(np.uint16),
                          y32.cpu().numpy()[:, cols].astype(np.float16).view(np.uint16))


@pytest.mark.gpu
@pytest.mark.parametrize("g", [128, 32768])
def test_quantize_2g_values(dev, g):
    """X of 65536 x 32768 fp16 (2^31 values, 4 GiB): a seeded 64-row block
    repeated on the GPU, so that each row's codes and scales are those of
    its source row; rows on both sides of the 2^31-byte offset checked."""
    M, K = 65536, 32768
    x0, _ = inputs.problem(64, 8, K, seed=g, act="outlier")
    x = torch.from_numpy(x0).to(dev).repeat(M // 64, 1)
    qa, sa = apex4.quantize_act(x, g)
    torch.cuda.synchronize()
    del x
    oq, os_ = orc.quantize(x0, g)
    for r in (0, 63, 32767, 32768, 32769, 50000, 65535):
        assert np.array_equal(qa[r].cpu().numpy(), oq[r % 64]), r
        assert np.array_equal(sa[r].cpu().numpy().view(np.uint32), os_[r % 64].view(np.uint32)), r
