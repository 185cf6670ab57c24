"""Graph capture of the hot path.

bench.py times replays of one captured HIP graph per step (activation
quantization + GEMM per layer).  A replay must give exactly the eager result:
here the step is captured once, then replayed four times, each time after
eager work that changes the input and recomputes the eager reference; every
replay is compared bit for bit with that reference (the kernels are
deterministic, so eager and replayed launches must agree exactly).
"""
import numpy as np
import pytest

from w4a4_group_quantized_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from w4a4_group_quantized_amd import apex4
    apex4.lib()
    return torch.device("cuda:0")


# decode-shaped (weight-streaming kernel), prefill-shaped with g = 128 and with
# one group over K (tiled kernels), small groups (step-major tiled kernel)
@pytest.mark.parametrize("M,N,K,g", [(16, 1024, 1024, 128), (300, 384, 1024, 128),
                                     (300, 384, 1024, 1024), (300, 384, 1024, 32)])
def test_graph_replays_match_eager(dev, M, N, K, g):
    import torch
    from w4a4_group_quantized_amd import apex4

    x, w = inputs.problem(M, N, K, seed=7, act="outlier")
    tx = torch.from_numpy(np.array(x)).to(dev)
    qw, sw = apex4.pack_weight(torch.from_numpy(np.array(w)).to(dev), g)
    qa = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    sa = torch.empty((M, K // g), dtype=torch.float32, device=dev)
    y = torch.empty((M, N), dtype=torch.float16, device=dev)

    def step():
        apex4.quantize_act(tx, g, out=(qa, sa))
        apex4.gemm(qa, sa, g, qw, sw, g, K, y16=y)

    step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=torch.cuda.Stream()):
        step()
    torch.cuda.synchronize()

    base = tx.clone()
    for rep in range(4):
        # eager work between replays: a new input, and its eager result
        tx.copy_(base * (1.0 + 0.25 * rep))
        step()
        torch.cuda.synchronize()
        ref_y, ref_qa, ref_sa = y.clone(), qa.clone(), sa.clone()
        y.fill_(0.0)
        qa.fill_(0)
        sa.fill_(0.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(qa, ref_qa), rep
        assert torch.equal(sa, ref_sa), rep
        assert torch.equal(y, ref_y), rep
