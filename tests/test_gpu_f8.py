"""The FP8-coded variant (apex4_quantize_f8, apex4_gemm_w4a4_f8) against the
CPU oracle and against the INT4 path.

The codes are the quantization rule's INT4 codes written as E4M3 bytes, so
the bar is: every byte decodes (E4M3: sign, 4 exponent bits with bias 7, 3
mantissa bits, exponent 0 subnormal) to exactly the oracle's code, scales
bit-exact; per-group sums P exact; fp32 output within 1e-5 of max|Y_ref|
and fp16 within one ulp of fp16(Y_ref).  Against the INT4 path the fp32
output is bit-identical: both add the same S_j * P_j in the same order (the
INT4 path's 2^-8 on S and 2^8 on P are exact powers of two).
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


def e4m3_value(b):
    """E4M3 (OCP) byte -> float, from the format's definition (finite values)."""
    b = np.asarray(b, dtype=np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = b & 0x7
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7))
    return sign * val


def unpack_codes(q):
    """oracle packed nibbles [rows, K/2] -> int codes [rows, K] (low nibble first)"""
    lo = (q & 0xF).astype(np.int8)
    hi = (q >> 4).astype(np.int8)
    lo = np.where(lo > 7, lo - 16, lo)
    hi = np.where(hi > 7, hi - 16, hi)
    out = np.empty((q.shape[0], q.shape[1] * 2), dtype=np.int8)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out


def test_e4m3_decoder_pins():
    # the integers -8..7 in E4M3: 1.0 = 0x38, 7 = 0x4E, -8 = 0xD0, 0.5 = 0x30
    assert list(e4m3_value([0x00, 0x38, 0x40, 0x44, 0x4E, 0xD0, 0x30, 0xB8])) == [0, 1, 2, 3, 7, -8, 0.5, -1]


@pytest.mark.gpu
@pytest.mark.parametrize("g", [64, 128])
@pytest.mark.parametrize("kind", inputs.ACT_KINDS)
@pytest.mark.parametrize("rows,K", [(1, 128), (37, 1152), (300, 4096)])
def test_quantize_f8_codes(dev, kind, rows, K, g):
    x, _ = inputs.problem(rows, 8, K, seed=rows + K, act=kind)
    q8, s = apex4.quantize_f8(torch.from_numpy(x).to(dev), g)
    torch.cuda.synchronize()
    oq, os_ = orc.quantize(x, g)
    codes = unpack_codes(oq)
    got = e4m3_value(q8.cpu().numpy())
    assert np.array_equal(got, codes.astype(np.float64))
    assert np.array_equal(s.cpu().numpy().view(np.uint32), os_.view(np.uint32))
    assert not np.any(q8.cpu().numpy() == 0x80)          # no -0


def run_f8(dev, x, w, rows=None, want_p=True, g=128):
    tx, tw = torch.from_numpy(x).to(dev), torch.from_numpy(w).to(dev)
    qa8, sa = apex4.quantize_f8(tx, g)
    qw8, sw = apex4.quantize_f8(tw, g)
    y16, y32, ps = apex4.gemm_f8(qa8, sa, qw8, sw, g, want_y32=True, want_psum=want_p)
    torch.cuda.synchronize()
    K = x.shape[1]
    oqa, osa = orc.quantize(x, g)
    oqw, osw = orc.quantize(w, g)
    r = np.arange(x.shape[0]) if rows is None else rows
    _, o32, op = orc.gemm(oqa[r], osa[r], g, oqw, osw, g, K, want_p=want_p)
    y32n, y16n = y32.cpu().numpy()[r], y16.cpu().numpy()[r]
    scale = float(np.abs(o32).max())
    tol = REL_TOL * max(scale, 1e-30)
    assert float(np.abs(y32n.astype(np.float64) - o32).max()) <= tol
    assert np.array_equal(y16n.view(np.uint16), y32n.astype(np.float16).view(np.uint16))
    r16 = o32.astype(np.float16)
    ulp = np.spacing(np.abs(r16)).astype(np.float64)
    assert np.all(np.abs(y16n.astype(np.float64) - r16.astype(np.float64)) <= ulp + tol)
    if want_p:
        assert np.array_equal(ps.cpu().numpy()[r], op)
    return tx, tw, y32


@pytest.mark.gpu
@pytest.mark.parametrize("g", [64, 128])
@pytest.mark.parametrize("M,N,K", [(16, 1024, 1024), (300, 300, 384), (257, 130, 1152), (513, 257, 2048)])
def test_gemm_f8_matches_oracle(dev, M, N, K, g):
    """Ragged M and N, odd stage counts (3 and 9 stages of 128 codes: one
    group of 128 or two of 64 each)."""
    x, w = inputs.problem(M, N, K, seed=71 + M, act="outlier")
    run_f8(dev, x, w, g=g)


@pytest.mark.gpu
@pytest.mark.parametrize("g", [64, 128])
def test_gemm_f8_equals_int4_path(dev, g):
    # a whole number of rounds of 256x128 tiles (512 x 64 CUs columns), so the
    # INT4 path runs over all of K in every tile, with no K split, and both
    # add the groups in the same order
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    x, w = inputs.problem(512, 64 * cus, 2048, seed=5, act="student_t")
    rows = np.array([0, 1, 255, 256, 300, 511])
    tx, tw, y32 = run_f8(dev, x, w, rows=rows, g=g)
    qa, sa = apex4.quantize_act(tx, g)
    qw, sw = apex4.pack_weight(tw, g)
    assert apex4.workspace_size(512, 64 * cus, 2048, g, g) == 0
    _, y32i, _ = apex4.gemm(qa, sa, g, qw, sw, g, 2048, want_y32=True)
    torch.cuda.synchronize()
    assert torch.equal(y32.view(torch.int32), y32i.view(torch.int32))


@pytest.mark.gpu
def test_gemm_f8_full_7b_qkv(dev):
    x, w = inputs.problem(2048, 12288, 4096, seed=0, act="outlier")
    rows = np.array([0, 1, 255, 256, 1023, 1500, 2046, 2047])
    run_f8(dev, x, w, rows=rows, want_p=False)


@pytest.mark.gpu
def test_f8_argument_checks(dev):
    x = torch.zeros((4, 256), dtype=torch.float16, device=dev)
    with pytest.raises(apex4.Apex4Error):
        apex4.quantize_f8(x, 32)                          # groups of 64 and 128 only
    q8 = torch.zeros((4, 200), dtype=torch.uint8, device=dev)
    s = torch.ones((4, 1), dtype=torch.float32, device=dev)
    with pytest.raises(apex4.Apex4Error):
        apex4.gemm_f8(q8, s, q8, s)                      # K = 200 is not a multiple of 128
    q8 = torch.zeros((4, 256), dtype=torch.uint8, device=dev)
    s = torch.ones((4, 8), dtype=torch.float32, device=dev)
    with pytest.raises(apex4.Apex4Error):
        apex4.gemm_f8(q8, s, q8, s)                      # groups of 32: no FP8 kernel
