"""W4A4Linear and the synthetic LLaMA-shaped layer (w4a4_group_quantized_amd/linear.py)
against the CPU oracle.

The module runs apex4_linear_w4a4; the bar is the one of
the GEMM parity tests: packed weight codes and scales bit-exact, fp16 output
within one fp16 ulp (plus 1e-5 of max|Y_ref|) of fp16(Y_ref).  In the layer,
every linear is checked on the fp16 input it actually received (the torch
ops between the linears are not part of the method and are not checked
against the oracle).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import oracle as orc  # noqa: E402
from w4a4_group_quantized_amd import apex4, inputs  # noqa: E402
from w4a4_group_quantized_amd.linear import LlamaLayerW4A4, W4A4Linear  # noqa: E402

REL_TOL = 1e-5


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    apex4.lib()   # raises when the HIP library is missing: no fallback
    return torch.device("cuda:0")


def check_y16(y16, r32):
    tol = REL_TOL * max(float(np.abs(r32).max()), 1e-30)
    r16 = r32.astype(np.float16)
    ulp = np.spacing(np.abs(r16)).astype(np.float64)
    d16 = np.abs(y16.astype(np.float64) - r16.astype(np.float64))
    assert np.all(d16 <= ulp + tol), float((d16 / (ulp + tol)).max())


def oracle_linear(x, w, ga, gw):
    K = x.shape[1]
    qa, sa = orc.quantize(x, ga)
    qw, sw = orc.quantize(w, gw)
    _, r32, _ = orc.gemm(qa, sa, ga, qw, sw, gw, K)
    return qw, sw, r32


@pytest.mark.gpu
@pytest.mark.parametrize("M,K,N,ga,gw", [(37, 512, 384, 128, 128), (5, 1024, 256, 128, 1024),
                                         (64, 768, 640, 64, 64)])
def test_linear_matches_oracle(dev, M, K, N, ga, gw):
    x, w = inputs.problem(M, N, K, seed=M + K, act="outlier")
    lin = W4A4Linear.from_weight(torch.from_numpy(w).to(dev), gw, ga)
    y = lin(torch.from_numpy(x).to(dev))
    y2 = lin(torch.from_numpy(x).to(dev))          # buffers reused at the same row count
    torch.cuda.synchronize()
    qw, sw, r32 = oracle_linear(x, w, ga, gw)
    assert np.array_equal(lin.qw.cpu().numpy(), qw)
    assert np.array_equal(lin.sw.cpu().numpy().view(np.uint32), sw.view(np.uint32))
    check_y16(y.cpu().numpy(), r32)
    assert torch.equal(y, y2)


@pytest.mark.gpu
def test_linear_leading_dims_and_new_row_counts(dev):
    x, w = inputs.problem(2 * 7, 256, 512, seed=11, act="normal")
    lin = W4A4Linear.from_weight(torch.from_numpy(w).to(dev), 128)
    tx = torch.from_numpy(x).to(dev)
    y3 = lin(tx.view(2, 7, 512))
    assert y3.shape == (2, 7, 256)
    y1 = lin(tx[:3])                                 # another row count: its own buffers
    torch.cuda.synchronize()
    _, _, r32 = oracle_linear(x, w, 128, 128)
    check_y16(y3.reshape(14, 256).cpu().numpy(), r32)
    check_y16(y1.cpu().numpy(), r32[:3])
    with pytest.raises(ValueError):
        lin(tx[:, :256])


@pytest.mark.gpu
@pytest.mark.parametrize("M", [1, 24])
def test_linear_out_buffer_and_strided_input(dev, M):
    """`out=` is written in place and returned; a non-contiguous input (every
    other column of a wider tensor) gives the bits of its contiguous copy."""
    x, w = inputs.problem(M, 384, 512, seed=21 + M, act="outlier")
    lin = W4A4Linear.from_weight(torch.from_numpy(w).to(dev), 128)
    wide = torch.zeros((M, 1024), dtype=torch.float16, device=dev)
    wide[:, ::2] = torch.from_numpy(x).to(dev)
    view = wide[:, ::2]
    assert not view.is_contiguous()
    out = torch.empty((M, 384), dtype=torch.float16, device=dev)
    y = lin(view, out=out)
    ref = lin(view.contiguous())
    torch.cuda.synchronize()
    assert y.data_ptr() == out.data_ptr()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    _, _, r32 = oracle_linear(x, w, 128, 128)
    check_y16(out.cpu().numpy(), r32)


@pytest.mark.gpu
@pytest.mark.parametrize("M", [40, 3])
def test_layer_every_linear_matches_oracle(dev, M):
    hidden, inter, g = 256, 384, 128
    layer = LlamaLayerW4A4.random(hidden, inter, g, seed=3, device=dev)
    # the same weights, regenerated on the host in the same draw order
    rng = np.random.default_rng(3)
    shapes = {"qkv": (3 * hidden, hidden), "o": (hidden, hidden),
              "gate_up": (2 * inter, hidden), "down": (hidden, inter)}
    ws = {n: inputs.weights(rng, *shapes[n]) for n in LlamaLayerW4A4.NAMES}
    x = inputs.activations(np.random.default_rng(7), M, hidden, "outlier", 7)
    out, seen = layer(torch.from_numpy(x).to(dev), return_inputs=True)
    torch.cuda.synchronize()
    assert out.shape == (M, hidden) and bool(torch.isfinite(out).all())
    for name, (xi, yi) in zip(LlamaLayerW4A4.NAMES, seen):
        qw, _, r32 = oracle_linear(xi.cpu().numpy(), ws[name], g, g)
        assert np.array_equal(getattr(layer, name).qw.cpu().numpy(), qw), name
        check_y16(yi.cpu().numpy(), r32)
    assert layer.linear_shapes() == [(256, 768), (256, 256), (256, 768), (384, 256)]


@pytest.mark.gpu
@pytest.mark.parametrize("ga,gw", [(128, 128), (256, 256), (128, "K"), (64, 64), ("K", "K")])
@pytest.mark.parametrize("M", [1, 2, 3, 16, 300])
def test_linear_entry_equals_quantize_then_gemm(dev, M, ga, gw):
    """apex4_linear_w4a4 gives the bits of apex4_quantize_act followed by
    apex4_gemm_w4a4 (fp16 and fp32 outputs); with 1-2 rows, groups of 128
    or 256 and K <= 8192 the decode kernel quantizes the rows itself and needs
    no workspace."""
    K, N = 1024, 1000
    ga = K if ga == "K" else ga
    gw = K if gw == "K" else gw
    x, w = inputs.problem(M, N, K, seed=M * 7 + ga, act="outlier")
    tx, tw = torch.from_numpy(x).to(dev), torch.from_numpy(w).to(dev)
    qw, sw = apex4.pack_weight(tw, gw)
    need = apex4.linear_workspace_size(M, N, K, ga, gw)
    fused = M <= 2 and ga in (128, 256)
    assert (need == 0) == fused
    y16, y32 = apex4.linear(tx, ga, qw, sw, gw, want_y32=True)
    y16b, y32b = apex4.linear(tx, ga, qw, sw, gw, want_y32=True)
    qa, sa = apex4.quantize_act(tx, ga)
    r16, r32, _ = apex4.gemm(qa, sa, ga, qw, sw, gw, K, want_y32=True)
    torch.cuda.synchronize()
    assert torch.equal(y32.view(torch.int32), r32.view(torch.int32))
    assert torch.equal(y16.view(torch.int16), r16.view(torch.int16))
    assert torch.equal(y32.view(torch.int32), y32b.view(torch.int32))
    if M <= 16:
        _, _, o32 = oracle_linear(x, w, ga, gw)
        check_y16(y16.cpu().numpy(), o32)


@pytest.mark.gpu
@pytest.mark.parametrize("M", [1, 2])
def test_linear_large_k_two_launches(dev, M):
    """K = 9216 > 8192: quantization into the workspace, then the GEMM; the
    same bits as the two calls."""
    K, N = 9216, 520
    x, w = inputs.problem(M, N, K, seed=M, act="student_t")
    tx, tw = torch.from_numpy(x).to(dev), torch.from_numpy(w).to(dev)
    qw, sw = apex4.pack_weight(tw, 128)
    assert apex4.linear_workspace_size(M, N, K, 128, 128) > 0
    y16, y32 = apex4.linear(tx, 128, qw, sw, 128, want_y32=True)
    qa, sa = apex4.quantize_act(tx, 128)
    r16, r32, _ = apex4.gemm(qa, sa, 128, qw, sw, 128, K, want_y32=True)
    torch.cuda.synchronize()
    assert torch.equal(y32.view(torch.int32), r32.view(torch.int32))
    assert torch.equal(y16.view(torch.int16), r16.view(torch.int16))


@pytest.mark.gpu
def test_linear_fused_full_70b_decode(dev):
    """The fused decode launch at the 70B up-projection shape (M=1, K=8192,
    N=28672), sampled output columns against the oracle."""
    M, K, N = 1, 8192, 28672
    x, w = inputs.problem(M, N, K, seed=4, act="outlier")
    tx, tw = torch.from_numpy(x).to(dev), torch.from_numpy(w).to(dev)
    qw, sw = apex4.pack_weight(tw, 128)
    y16, y32 = apex4.linear(tx, 128, qw, sw, 128, want_y32=True)
    torch.cuda.synchronize()
    cols = np.array([0, 1, 63, 64, 4095, 15000, 28670, 28671])
    oqa, osa = orc.quantize(x, 128)
    oqw, osw = orc.quantize(w[cols], 128)
    _, o32, _ = orc.gemm(oqa, osa, 128, oqw, osw, 128, K)
    got = y32.cpu().numpy()[:, cols].astype(np.float64)
    assert float(np.abs(got - o32).max()) <= REL_TOL * float(np.abs(o32).max())


@pytest.mark.gpu
def test_linear_argument_checks(dev):
    x = torch.zeros((40, 256), dtype=torch.float16, device=dev)
    qw = torch.zeros((64, 128), dtype=torch.uint8, device=dev)
    sw = torch.ones((64, 2), dtype=torch.float32, device=dev)
    small = torch.empty(16, dtype=torch.uint8, device=dev)
    with pytest.raises(apex4.Apex4Error):
        apex4.linear(x, 128, qw, sw, 128, workspace=small)        # workspace too small
    with pytest.raises(apex4.Apex4Error):
        apex4.linear(x, 96, qw, sw, 96)                           # unsupported group
    assert apex4.linear_workspace_size(40, 64, 256, 128, 128) > 0
    assert apex4.linear_workspace_size(1, 64, 256, 128, 128) == 0
    assert apex4.linear_workspace_size(1, 64, 200, 128, 128) == 0   # invalid: 0, and the call refuses
    assert apex4.linear_workspace_size(1, 64, 16384, 128, 128) > 0  # K > 8192: two launches


def test_linear_refuses_host_tensors():
    """No CPU path: the module takes GPU-packed weights only (host logic, no GPU needed)."""
    qw = torch.zeros((8, 64), dtype=torch.uint8)
    sw = torch.ones((8, 1), dtype=torch.float32)
    with pytest.raises(ValueError):
        W4A4Linear(qw, sw, 128)


@pytest.mark.gpu
@pytest.mark.parametrize("M", [16, 1])
def test_layer_graph_replays_match_eager(dev, M):
    """The layer forward captured as one HIP graph: every replay, with eager
    work and synchronizations between them, gives the eager result bit for bit
    (M = 1: every linear is one fused launch)."""
    layer = LlamaLayerW4A4.random(256, 384, 128, seed=5, device=dev)
    x = torch.from_numpy(inputs.activations(np.random.default_rng(9), M, 256, "outlier", 9)).to(dev)
    ref = layer(x).clone()                      # eager (also allocates the activation buffers)
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        out = layer(x)
    for r in range(4):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), r
        other = layer(x * 0.5)                  # eager work on the same buffers between replays
        torch.cuda.synchronize()
        assert not torch.equal(other, ref)
