"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar: packed codes, scales and per-group int32 sums bit-exact; fp32 output
within 1e-5 of max|Y_ref| (the fp32 summation order on the GPU is free); fp16
output within one fp16 ulp of fp16(Y_ref).  Small shapes are compared in full;
the full-size workloads (7B/70B-shaped prefill layers, 70B decode shapes, the
granularity sweep) are compared on sampled rows (every output row is
independent) with quantization checked on every row.
"""
import functools

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import oracle as orc  # noqa: E402
from w4a4_group_quantized_amd import apex4, inputs  # noqa: E402

pytestmark = pytest.mark.gpu
REL_TOL = 1e-5


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    apex4.lib()   # raises when the HIP library is missing: no fallback
    return torch.device("cuda:0")


def to_dev(a, dev):
    return torch.from_numpy(np.array(a, copy=True, order="C")).to(dev)


def check_y(y32, y16, r32):
    """fp32 within REL_TOL of max|ref|; fp16 is the RNE rounding of the kernel's
    own fp32 result, hence within one fp16 ulp plus the fp32 tolerance of
    fp16(ref) (near zero the fp16 grid is finer than the fp32 tolerance)."""
    scale = float(np.abs(r32).max())
    tol = REL_TOL * max(scale, 1e-30)
    err = float(np.abs(y32.astype(np.float64) - r32.astype(np.float64)).max())
    assert err <= tol, (err, scale)
    with np.errstate(over="ignore"):
        assert np.array_equal(y16.view(np.uint16), y32.astype(np.float16).view(np.uint16))
        r16 = r32.astype(np.float16)
    fin = np.isfinite(r16)
    assert np.array_equal(y16[~fin], r16[~fin])     # overflow to +-inf on both sides
    ulp = np.spacing(np.abs(r16[fin])).astype(np.float64)
    d16 = np.abs(y16[fin].astype(np.float64) - r16[fin].astype(np.float64))
    assert np.all(d16 <= ulp + tol), float((d16 / (ulp + tol)).max())
    return err / max(scale, 1e-30)


def gpu_quantize(x, g, dev, weight=False):
    fn = apex4.pack_weight if weight else apex4.quantize_act
    q, s = fn(to_dev(x, dev), g)
    torch.cuda.synchronize()
    return q, s


def run_case(dev, x, w, ga, gw, rows=None, want_p=False, p_rows=None):
    """Quantize X and pack W on the GPU, run the GEMM, compare everything.

    rows: the output rows compared (None: all).  want_p: the per-group int32
    sums are compared bit for bit, on `rows` (the GPU writes them for every
    row), or, with p_rows = (row0, step, count), on rows row0 + i * step
    only, which is all the GPU writes (apex4_gemm_w4a4_debug, in the launch
    configuration of apex4_gemm_w4a4); those rows are compared for Y too.
    """
    M, K = x.shape
    tqa, tsa = gpu_quantize(x, ga, dev)
    tqw, tsw = gpu_quantize(w, gw, dev, weight=True)
    oqa, osa = orc.quantize(x, ga)
    oqw, osw = orc.quantize(w, gw)
    assert np.array_equal(tqa.cpu().numpy(), oqa)
    assert np.array_equal(tsa.cpu().numpy().view(np.uint32), osa.view(np.uint32))
    assert np.array_equal(tqw.cpu().numpy(), oqw)
    assert np.array_equal(tsw.cpu().numpy().view(np.uint32), osw.view(np.uint32))
    y16, y32, ps = apex4.gemm(tqa, tsa, ga, tqw, tsw, gw, K, want_y32=True, want_psum=want_p,
                              psum_rows=p_rows)
    torch.cuda.synchronize()
    r = np.arange(M) if rows is None else np.asarray(rows)
    prow = None
    if p_rows is not None:
        row0, step, count = p_rows
        prow = row0 + step * np.arange(count)
        r = np.unique(np.concatenate([r, prow]))
    o16, o32, op = orc.gemm(oqa[r], osa[r], ga, oqw, osw, gw, K, want_p=want_p)
    rel = check_y(y32.cpu().numpy()[r], y16.cpu().numpy()[r], o32)
    if want_p:
        gp = ps.cpu().numpy()
        if prow is None:
            assert np.array_equal(gp[r], op)
        else:
            assert np.array_equal(gp, op[np.searchsorted(r, prow)])
    return rel


def tile_rows(M, row0):
    """(row0, 256, count): one row in every 256-row tile of the tiled kernels."""
    return (row0, 256, (M - 1 - row0) // 256 + 1)


@functools.lru_cache(maxsize=1)
def big_problem(M, N, K, act):
    """Full-size inputs (cached: the sweep's six cases share one draw)."""
    x, w = inputs.problem(M, N, K, seed=0, act=act)
    x.setflags(write=False)
    w.setflags(write=False)
    return x, w


def sample_rows(M, n=16, seed=0):
    rng = np.random.default_rng(seed)
    r = set(np.linspace(0, M - 1, n // 2).astype(int).tolist())
    r |= set(rng.choice(M, size=min(M, n // 2), replace=False).tolist())
    return np.array(sorted(r))


# ------------------------------------------------------------- quantization


@pytest.mark.parametrize("g", [32, 64, 128, 256, "K"])
@pytest.mark.parametrize("kind", inputs.ACT_KINDS)
@pytest.mark.parametrize("M,K", [(1, 1024), (37, 1152), (64, 4096)])
def test_quantize_bitexact(dev, g, kind, M, K):
    g = K if g == "K" else g
    if K % g:
        pytest.skip("group does not divide K")
    rng = np.random.default_rng(M * 7 + K)
    x = inputs.activations(rng, M, K, kind, seed=M)
    x[M // 2, :g] = 0                       # an all-zero group
    x[0, -8:] = np.float16(3e-7)            # fp16 subnormals
    q, s = gpu_quantize(x, g, dev)
    oq, os_ = orc.quantize(x, g)
    assert np.array_equal(q.cpu().numpy(), oq)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), os_.view(np.uint32))


def test_quantize_hand_cases_on_gpu(dev):
    """The hand-worked tie/scale cases in tests/golden, through the GPU kernel."""
    from tests.test_oracle_pins import _read_quant_cases
    for c in _read_quant_cases():
        vals = [float(v) for v in c["x"]]
        x = np.zeros((1, 32), np.float16)
        x[0, :len(vals)] = vals
        q, s = gpu_quantize(x, 32, dev)
        assert s.cpu().numpy()[0, 0].view(np.uint32) == int(c["scale"][0], 16)
        codes = orc.codes(q.cpu().numpy(), 32)[0, :len(vals)]
        assert codes.tolist() == [int(v) for v in c["codes"]]


def test_quantize_empty_is_noop(dev):
    x = torch.empty((0, 256), dtype=torch.float16, device=dev)
    q, s = apex4.quantize_act(x, 128)
    assert q.shape == (0, 128) and s.shape == (0, 2)


# ------------------------------------------------------------- GEMM, small


@pytest.mark.parametrize("g", [32, 64, 128, 256, 1024])
def test_gemm_tiny_config(dev, g):
    """M=16, K=N=1024, X~N(0,1), W~N(0,0.02), seed 0: everything compared, P included."""
    x, w = inputs.problem(16, 1024, 1024, seed=0, act="normal")
    run_case(dev, x, w, g, g, want_p=True)


@pytest.mark.parametrize("M", [40, 300])
@pytest.mark.parametrize("ga", [32, 64, 128, 256])
def test_gemm_mixed_mode_small(dev, ga, M):
    """Per-channel weight scales with grouped activations: 40 rows take the
    weight-streaming kernel, 300 rows (two row tiles, ragged) a tiled one."""
    x, w = inputs.problem(M, 200, 1024, seed=3, act="outlier")
    run_case(dev, x, w, ga, 1024, want_p=True)


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (1, 8, 256), (3, 130, 384), (129, 129, 1152),
                                   (200, 77, 512), (130, 260, 2048)])
@pytest.mark.parametrize("g", [32, 128, "K"])
def test_gemm_ragged_shapes(dev, M, N, K, g):
    g = K if g == "K" else g
    x, w = inputs.problem(M, N, K, seed=M + N, act="normal")
    run_case(dev, x, w, g, g, want_p=True)


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8, 16, 17, 32, 33, 64])
@pytest.mark.parametrize("ga,gw", [(128, 128), (256, 256), ("K", "K"), (128, "K")])
@pytest.mark.parametrize("K", [2048, 9216])
def test_gemm_decode_rows(dev, M, ga, gw, K):
    """The decode kernels: 1-2 rows the row-streaming dot8 kernel (K = 2048
    leaves most lanes without a unit, K = 9216 = 72 units gives lanes a second,
    partial pass); 3-16 rows the LDS-streaming MFMA kernel (4, 8 or 16
    activation rows held; K = 9216 ends in half an item); 17-64 rows its
    K-outer variant (2 or 4 row tiles).  N = 300 is not a multiple of 16 or of
    the wave count; group sums P are compared too."""
    ga = K if ga == "K" else ga
    gw = K if gw == "K" else gw
    x, w = inputs.problem(M, 300, K, seed=11 + M, act="outlier")
    run_case(dev, x, w, ga, gw, want_p=True)


@pytest.mark.parametrize("M,N,K", [(300, 300, 1024), (260, 130, 2560), (513, 257, 3328), (65, 1000, 1152),
                                   (1024, 512, 4096)])
@pytest.mark.parametrize("ga,gw", [(64, 64), (64, "K"), (32, 32)])
def test_gemm_groups_within_a_stage(dev, M, N, K, ga, gw):
    """Groups of 64 and 32 on the ping-pong tiled kernel: two or four groups
    per 128-value stage, each with its own matrix phase, scale products and
    rescale; 9, 20, 26 and 32 stages (odd and even loop ends), ragged M and
    N, a single mostly empty row tile (65 rows); also mixed mode with
    activation groups of 64 (per-channel weight scales)."""
    gw = K if gw == "K" else gw
    x, w = inputs.problem(M, N, K, seed=43 + M, act="outlier")
    run_case(dev, x, w, ga, gw, want_p=True)


@pytest.mark.parametrize("M,N,K", [(300, 300, 1024), (260, 130, 2560), (513, 257, 3328)])
@pytest.mark.parametrize("ga,gw", [(256, 256), (256, "K")])
def test_gemm_groups_of_two_stages(dev, M, N, K, ga, gw):
    """Groups of 256 (and mixed mode with activation groups of 256) on the
    ping-pong tiled kernel: a group spans two 128-value stages, so the int32
    sums run across a stage boundary before the rescale; 10 and 13 groups
    (odd), ragged M and N."""
    gw = K if gw == "K" else gw
    x, w = inputs.problem(M, N, K, seed=41 + M, act="outlier")
    run_case(dev, x, w, ga, gw, want_p=True)


@pytest.mark.parametrize("M,N,K", [(24, 9000, 4224), (64, 9000, 4224), (48, 5000, 2048), (12, 9000, 20480),
                                   (4, 9000, 36864), (4, 3000, 40960), (16, 9000, 10240), (8, 5000, 20480),
                                   (3, 2000, 40960)])
@pytest.mark.parametrize("ga,gw", [(128, 128), (128, "K")])
def test_gemm_decode_many_blocks(dev, M, N, K, ga, gw):
    """Decode shapes with several 16-column blocks per workgroup: the K-outer
    kernel with groups of 4 blocks (24 rows, 563 blocks) and of 2 (64 and 48
    rows, the last group half empty at 9000 columns), K = 4224 ending in a
    128-value item; the LDS-streaming kernel with the activation rows brought
    per item because they do not fit whole (12 rows of K = 20480, 4 and 3
    rows of K = 40960, 16 rows of K = 10240, 8 rows of K = 20480), and held
    whole when they just fit (4 rows of K = 36864)."""
    ga = K if ga == "K" else ga
    gw = K if gw == "K" else gw
    x, w = inputs.problem(M, N, K, seed=31 + M, act="outlier")
    run_case(dev, x, w, ga, gw, want_p=True)


@pytest.mark.parametrize("M,g", [(1, 128), (2, 256), (8, 128), (13, "K"), (40, 128), (40, 256), (64, "K"),
                                 (300, 128), (300, 256), (300, "K"), (300, 32), (520, 64), (17, 64)])
def test_gemm_debug_rows(dev, M, g):
    """apex4_gemm_w4a4_debug keeps the group sums of every p_step-th row from
    p_row0: each kernel (row-streaming, LDS-streaming, K-outer, skinny,
    ping-pong, step-major tiled) against the oracle.  The buffer is exactly
    [count, N, G], so a sum of any other row written into it would overwrite
    a kept row's entry and show as a mismatch."""
    K = 1024
    g = K if g == "K" else g
    x, w = inputs.problem(M, 200, K, seed=5 + M, act="outlier")
    row0 = M // 3
    step = max(1, M // 5)
    count = (M - 1 - row0) // step + 1
    run_case(dev, x, w, g, g, rows=sample_rows(M, n=4), want_p=True, p_rows=(row0, step, count))


@pytest.mark.parametrize("M", [300, 520])
def test_gemm_debug_rows_step_major(dev, M):
    """The same for the step-major tiled kernel, which runs mixed mode with
    activation groups of 32 (per-channel weight scales): the kept rows' group
    sums against the oracle."""
    K = 1024
    x, w = inputs.problem(M, 200, K, seed=9 + M, act="outlier")
    row0 = M // 3
    step = max(1, M // 5)
    count = (M - 1 - row0) // step + 1
    run_case(dev, x, w, 32, K, rows=sample_rows(M, n=4), want_p=True, p_rows=(row0, step, count))


@pytest.mark.parametrize("g", [32, 64, 128, 256, 1024])
def test_gemm_unit_scales_integer_exact(dev, g):
    """Random packed codes (-8 included), all scales 1: Y is the exact integer matmul."""
    M, N, K = 70, 150, 1024
    qa, _ = inputs.random_packed(M, K, 1, seed=21)
    qw, _ = inputs.random_packed(N, K, 1, seed=22)
    sa = np.ones((M, K // g), np.float32)
    sw = np.ones((N, K // g), np.float32)
    y16, y32, ps = apex4.gemm(to_dev(qa, dev), to_dev(sa, dev), g, to_dev(qw, dev),
                              to_dev(sw, dev), g, K, want_y32=True, want_psum=True)
    torch.cuda.synchronize()
    o16, o32, op = orc.gemm(qa, sa, g, qw, sw, g, K, want_p=True)
    assert np.array_equal(y32.cpu().numpy(), o32)
    assert np.array_equal(ps.cpu().numpy(), op)
    assert np.array_equal(y16.cpu().numpy(), o16)


def test_gemm_random_scales_and_codes(dev):
    """Random packed codes with -8 and wide-ranging scales, mixed and equal modes."""
    M, N, K = 33, 96, 2048
    for ga, gw, seed in ((128, 128, 1), (64, 2048, 2), (2048, 2048, 3)):
        qa, sa = inputs.random_packed(M, K, K // ga, seed=seed, scale_lo=1e-5, scale_hi=0.05)
        qw, sw = inputs.random_packed(N, K, K // gw, seed=seed + 9, scale_lo=1e-5, scale_hi=0.05)
        y16, y32, ps = apex4.gemm(to_dev(qa, dev), to_dev(sa, dev), ga, to_dev(qw, dev),
                                  to_dev(sw, dev), gw, K, want_y32=True, want_psum=True)
        torch.cuda.synchronize()
        o16, o32, op = orc.gemm(qa, sa, ga, qw, sw, gw, K, want_p=True)
        assert np.array_equal(ps.cpu().numpy(), op)
        check_y(y32.cpu().numpy(), y16.cpu().numpy(), o32)


def test_gemm_without_optional_outputs(dev):
    """y16 alone (no fp32, no debug sums) matches the run with them."""
    x, w = inputs.problem(64, 256, 1024, seed=4)
    qa, sa = gpu_quantize(x, 128, dev)
    qw, sw = gpu_quantize(w, 128, dev, weight=True)
    a = apex4.gemm(qa, sa, 128, qw, sw, 128, 1024)
    b, _, _ = apex4.gemm(qa, sa, 128, qw, sw, 128, 1024, want_y32=True, want_psum=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_gemm_empty_shapes(dev):
    z = torch.empty((0, 64), dtype=torch.uint8, device=dev)
    s0 = torch.empty((0, 1), dtype=torch.float32, device=dev)
    qw = torch.zeros((8, 64), dtype=torch.uint8, device=dev)
    sw = torch.ones((8, 1), dtype=torch.float32, device=dev)
    y = apex4.gemm(z, s0, 128, qw, sw, 128, 128)
    assert y.shape == (0, 8)


# ------------------------------------------------------------- full-size workloads


PREFILL_7B = [(4096, 12288), (4096, 4096), (4096, 22016), (11008, 4096)]
PREFILL_70B = [(8192, 10240), (8192, 8192), (8192, 57344), (28672, 8192)]
DECODE = [(8192, 28672), (28672, 8192)]


# Full sizes: Y on 16 sampled rows plus one row in every 256-row tile, whose
# per-group int32 sums are compared too (the debug sums of those rows only,
# from the same launch configuration as the plain call); decode shapes
# compare every row and every sum.


@pytest.mark.parametrize("K,N", PREFILL_7B)
def test_full_7b_prefill(dev, K, N):
    x, w = big_problem(2048, N, K, "outlier")
    run_case(dev, x, w, 128, 128, rows=sample_rows(2048), want_p=True, p_rows=tile_rows(2048, 101))


@pytest.mark.parametrize("K,N", DECODE)
@pytest.mark.parametrize("M", [1, 4, 16, 64])
def test_full_decode(dev, M, K, N):
    x, w = big_problem(M, N, K, "normal")
    run_case(dev, x, w, 128, 128, want_p=True)


@pytest.mark.parametrize("K,N", PREFILL_70B)
def test_full_70b_prefill(dev, K, N):
    x, w = big_problem(4096, N, K, "outlier")
    run_case(dev, x, w, 128, 128, rows=sample_rows(4096), want_p=True, p_rows=tile_rows(4096, 190))


@pytest.mark.parametrize("ga,gw", [(32, 32), (64, 64), (128, 128), (256, 256), (8192, 8192),
                                   (128, 8192)])
def test_full_granularity_sweep(dev, ga, gw):
    x, w = big_problem(8192, 28672, 8192, "student_t")
    run_case(dev, x, w, ga, gw, rows=sample_rows(8192), want_p=True, p_rows=tile_rows(8192, 37))


# ------------------------------------------------- K split of a partial last round


@pytest.mark.parametrize("M,N,K,ga,gw", [(300, 16640, 512, 128, 128), (257, 16512, 1152, 128, 128),
                                         (300, 16640, 1024, 128, 1024), (130, 1000, 4096, 128, 128),
                                         (300, 4096, 1024, 128, 128), (65, 640, 2048, 128, 2048),
                                         (300, 16640, 512, 64, 64), (257, 16512, 1152, 64, 64),
                                         (300, 16640, 1024, 64, 1024), (300, 16640, 512, 32, 32),
                                         (257, 16512, 1152, 32, 32)])
def test_gemm_split_last_round(dev, M, N, K, ga, gw):
    """Shapes whose last round of 256x128 output tiles (the only one, for few
    tiles) fills at most half the GPU's compute units: those tiles run as 2 to
    4 parts of K into the workspace (uneven parts when the stage count does
    not divide: K = 1152 is 9 stages) and a reduction writes their Y.  Rows of
    the split tiles and of the others are checked; on a GPU where the shape
    does not split the test still checks the result."""
    x, w = inputs.problem(M, N, K, seed=M + N, act="outlier")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tiles = -(-M // 256) * -(-N // 128)
    stages = K // 128
    ws = apex4.workspace_size(M, N, K, ga, gw)
    tail = tiles % cus
    if tail and 2 * tail <= cus and stages >= 4:
        parts = min(cus // tail, stages // 2, 4)
        assert ws == parts * tail * 256 * 128 * 4
    else:
        assert ws == 0
    rows = np.unique(np.concatenate([sample_rows(M, n=8), np.arange(M - 3, M), np.arange(256, min(M, 259))]))
    # the K parts write the group sums of their own groups
    run_case(dev, x, w, ga, gw, rows=rows, want_p=True)
    # the parts are added in a fixed order: a second call gives the same bits
    tqa, tsa = gpu_quantize(x, ga, dev)
    tqw, tsw = gpu_quantize(w, gw, dev, weight=True)
    a = apex4.gemm(tqa, tsa, ga, tqw, tsw, gw, K, want_y32=True)[1]
    b = apex4.gemm(tqa, tsa, ga, tqw, tsw, gw, K, want_y32=True)[1]
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_gemm_split_workspace_too_small(dev):
    M, N, K = 300, 16640, 512
    need = apex4.workspace_size(M, N, K, 128, 128)
    if need == 0:
        pytest.skip("this GPU's compute-unit count does not split the shape")
    qa = torch.zeros((M, K // 2), dtype=torch.uint8, device=dev)
    sa = torch.ones((M, K // 128), dtype=torch.float32, device=dev)
    qw = torch.zeros((N, K // 2), dtype=torch.uint8, device=dev)
    sw = torch.ones((N, K // 128), dtype=torch.float32, device=dev)
    y = torch.empty((M, N), dtype=torch.float16, device=dev)
    ws = torch.empty(need - 16, dtype=torch.uint8, device=dev)
    st = apex4.lib().apex4_gemm_w4a4(apex4._ptr(qa), apex4._ptr(sa), 128, apex4._ptr(qw), apex4._ptr(sw), 128,
                                     M, N, K, apex4._ptr(y), None, None, apex4._ptr(ws), need - 16,
                                     torch.cuda.current_stream().cuda_stream)
    assert st == 4   # APEX4_ERR_WORKSPACE, nothing launched


@pytest.mark.parametrize("M", [17, 40, 64])
@pytest.mark.parametrize("N,K", [(8192, 8192), (1000, 5248)])
@pytest.mark.parametrize("ga,gw", [(128, 128), (128, "K")])
def test_gemm_decode_split_k(dev, M, N, K, ga, gw):
    """17-64 rows with at most 2 column blocks per workgroup (N = 8192: 512
    blocks; N = 1000: 63): the K-outer kernel's two K halves (K = 5248: 6
    items, the last ragged) into the workspace, then the reduction."""
    gw = K if gw == "K" else gw
    ws = apex4.workspace_size(M, N, K, ga, gw)
    assert ws == 2 * M * N * 4
    x, w = inputs.problem(M, N, K, seed=61 + M, act="outlier")
    # (each half writes the group sums of its own groups)
    run_case(dev, x, w, ga, gw, rows=None if M <= 17 else sample_rows(M), want_p=True)
    # the two halves are added in a fixed order: a second call gives the same bits
    tqa, tsa = gpu_quantize(x, ga, dev)
    tqw, tsw = gpu_quantize(w, gw, dev, weight=True)
    a = apex4.gemm(tqa, tsa, ga, tqw, tsw, gw, K, want_y32=True)[1]
    b = apex4.gemm(tqa, tsa, ga, tqw, tsw, gw, K, want_y32=True)[1]
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
