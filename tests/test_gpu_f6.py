"""The FP6-coded variant (apex4_quantize_f6, apex4_gemm_w4a4_f6) against the
CPU oracle.

The codes are the quantization rule's INT4 codes written as 6-bit FP6 E2M3
fields, so the bar is: every field decodes (E2M3: sign bit, 2 exponent bits
with bias 1, 3 mantissa bits, exponent 0 subnormal) to exactly the oracle's
code divided by 8, scales bit-exact; per-group sums P exact; fp32 output
within 1e-5 of max|Y_ref| and fp16 within one ulp of fp16(Y_ref).
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


def e2m3_value(f):
    """6-bit FP6 E2M3 field -> float, from the format's definition."""
    f = np.asarray(f, dtype=np.int64)
    sign = np.where(f & 0x20, -1.0, 1.0)
    e = (f >> 3) & 0x3
    m = f & 0x7
    val = np.where(e == 0, m / 8.0, (1.0 + m / 8.0) * 2.0 ** (e - 1))
    return sign * val


def unpack_f6(q6):
    """row-major packed rows [rows, 3K/4] bytes -> 6-bit fields [rows, K]:
    field k at bits 6k .. 6k+5 of the row, little-endian."""
    q6 = np.asarray(q6, dtype=np.uint8)
    rows, nb = q6.shape
    K = nb * 4 // 3
    bits = np.unpackbits(q6, axis=1, bitorder="little")          # [rows, 8 * nb]
    bits = bits.reshape(rows, K, 6).astype(np.int64)
    return (bits << np.arange(6)).sum(axis=2)


def untile_f6(q6, rows, K):
    """apex4_quantize_f6's tiled layout -> row-major packed rows [rows, 3K/4]:
    tile (row block b, group j) at byte (b * G + j) * 6144, chunk q of row i
    of the block at + q * 1024 + i * 16."""
    G = K // 128
    nb = (rows + 63) // 64
    t = np.asarray(q6, dtype=np.uint8).reshape(nb, G, 6, 64, 16)
    return t.transpose(0, 3, 1, 2, 4).reshape(nb * 64, G * 96)[:rows]


def tile_f6(rowmajor):
    """row-major packed rows [rows, 3K/4] -> the tiled layout (padding rows zero)."""
    rows, nb_bytes = rowmajor.shape
    G = nb_bytes // 96
    nb = (rows + 63) // 64
    full = np.zeros((nb * 64, nb_bytes), np.uint8)
    full[:rows] = rowmajor
    return full.reshape(nb, 64, G, 6, 16).transpose(0, 2, 3, 1, 4).reshape(nb * 64, nb_bytes)


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


def test_e2m3_decoder_pins():
    # E2M3: 0x08 = 1.0 (e=1, m=0), 0x0F = 1.875, 0x07 = 0.875 (subnormal),
    # 0x10 = 2.0, 0x1F = 7.5 (largest), 0x28 = -1.0
    assert list(e2m3_value([0x00, 0x08, 0x0F, 0x07, 0x10, 0x1F, 0x28])) == [0, 1.0, 1.875, 0.875, 2.0, 7.5, -1.0]
    # the field (c < 0) << 5 | |c| is c / 8 for every INT4 code
    for c in range(-8, 8):
        f = (32 if c < 0 else 0) | abs(c)
        assert e2m3_value(f) * 8 == c


def test_unpack_f6_pin():
    # fields 1, 33, 7, 40 (codes 1, -1, 7, -8) packed by hand: 1 | 33 << 6 |
    # 7 << 12 | 40 << 18 = 0xA07841, little-endian bytes 41 78 A0
    row = np.zeros((1, 96), np.uint8)
    row[0, :3] = [0x41, 0x78, 0xA0]
    assert unpack_f6(row)[0, :4].tolist() == [1, 33, 7, 40]


def test_tiled_layout_pin():
    # 70 rows (two blocks, the second padded), K = 256 (two groups): byte 17
    # of row 66's group 1 is chunk 1, byte 1 of it; row 66 is row 2 of block
    # 1: tile (1 * 2 + 1) * 6144, + 1 * 1024 + 2 * 16 + 1
    rm = np.zeros((70, 192), np.uint8)
    rm[66, 96 + 17] = 0xAB
    t = tile_f6(rm)
    assert t.shape == (128, 192)
    flat = t.reshape(-1)
    assert flat[(1 * 2 + 1) * 6144 + 1 * 1024 + 2 * 16 + 1] == 0xAB and flat.sum() == 0xAB
    assert np.array_equal(untile_f6(t, 70, 256), rm)


@pytest.mark.gpu
@pytest.mark.parametrize("kind", inputs.ACT_KINDS)
@pytest.mark.parametrize("rows,K", [(1, 128), (37, 1152), (300, 4096)])
def test_quantize_f6_codes(dev, kind, rows, K):
    x, _ = inputs.problem(rows, 8, K, seed=rows + K, act=kind)
    x[rows // 2, :128] = 0                       # an all-zero group
    q6, s = apex4.quantize_f6(torch.from_numpy(x).to(dev), 128)
    torch.cuda.synchronize()
    oq, os_ = orc.quantize(x, 128)
    q = q6.cpu().numpy()
    fields = unpack_f6(untile_f6(q, rows, K))
    # the padding rows of the last block are zeros
    assert not np.any(untile_f6(q, (rows + 63) // 64 * 64, K)[rows:])
    assert np.array_equal(e2m3_value(fields) * 8, unpack_codes(oq).astype(np.float64))
    assert np.array_equal(s.cpu().numpy().view(np.uint32), os_.view(np.uint32))
    assert not np.any(fields == 0x20)            # no -0


def run_f6(dev, x, w, rows=None, want_p=True):
    tx, tw = torch.from_numpy(x).to(dev), torch.from_numpy(w).to(dev)
    qa6, sa = apex4.quantize_f6(tx, 128)
    qw6, sw = apex4.quantize_f6(tw, 128)
    y16, y32, ps = apex4.gemm_f6(qa6, sa, qw6, sw, want_y32=True, want_psum=want_p)
    torch.cuda.synchronize()
    K = x.shape[1]
    oqa, osa = orc.quantize(x, 128)
    oqw, osw = orc.quantize(w, 128)
    r = np.arange(x.shape[0]) if rows is None else rows
    _, o32, op = orc.gemm(oqa[r], osa[r], 128, oqw, osw, 128, K, want_p=want_p)
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
    return y32


@pytest.mark.gpu
@pytest.mark.parametrize("M,N,K", [(16, 1024, 1024), (300, 300, 384), (257, 130, 1152), (513, 257, 2048),
                                   (1, 8, 128), (65, 1000, 256)])
def test_gemm_f6_matches_oracle(dev, M, N, K):
    """Ragged M and N (row and column tiles partly past the end), 1 to 16
    groups (a group is one 128-code stage; 1 and 2 stages test the copies
    issued two stages ahead past the end of K)."""
    x, w = inputs.problem(M, N, K, seed=91 + M, act="outlier")
    run_f6(dev, x, w)


@pytest.mark.gpu
def test_gemm_f6_random_codes_with_minus_eight(dev):
    """Random packed INT4 codes, -8 included (outside the quantizer's output),
    re-coded as E2M3 fields on the host by the field definition, unit scales:
    Y is the exact integer matmul and P the integer group sums."""
    M, N, K = 70, 150, 1024
    qa, _ = inputs.random_packed(M, K, 1, seed=23)
    qw, _ = inputs.random_packed(N, K, 1, seed=24)

    def to_f6(q):
        c = unpack_codes(q).astype(np.int64)
        f = np.where(c < 0, 32, 0) | np.abs(c)
        bits = ((f[:, :, None] >> np.arange(6)) & 1).astype(np.uint8).reshape(q.shape[0], -1)
        return np.packbits(bits, axis=1, bitorder="little")
    qa6, qw6 = to_f6(qa), to_f6(qw)
    assert np.array_equal(unpack_f6(qa6), np.where(unpack_codes(qa) < 0, 32, 0) | np.abs(unpack_codes(qa)))
    qa6, qw6 = tile_f6(qa6), tile_f6(qw6)
    sa = np.ones((M, K // 128), np.float32)
    sw = np.ones((N, K // 128), np.float32)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    y16, y32, ps = apex4.gemm_f6(t(qa6), t(sa), t(qw6), t(sw), want_y32=True, want_psum=True)
    torch.cuda.synchronize()
    o16, o32, op = orc.gemm(qa, sa, 128, qw, sw, 128, K, want_p=True)
    assert np.array_equal(ps.cpu().numpy(), op)
    assert np.array_equal(y32.cpu().numpy(), o32)


@pytest.mark.gpu
def test_gemm_f6_split_last_round(dev):
    """A last round of 256x128 tiles filling at most half the GPU runs as K
    parts into the workspace (the split of apex4_gemm_w4a4 for groups of 128),
    each part writing the group sums of its own groups; a second call gives
    the same bits."""
    M, N, K = 300, 16640, 1024
    x, w = inputs.problem(M, N, K, seed=77, act="outlier")
    rows = np.unique(np.concatenate([np.arange(0, M, 37), np.arange(M - 3, M)]))
    a = run_f6(dev, x, w, rows=rows)
    b = run_f6(dev, x, w, rows=rows, want_p=False)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.gpu
def test_gemm_f6_full_70b_qkv(dev):
    """LLaMA-2-70B GQA QKV prefill layer (M=4096, K=8192, N=10240), one row in
    every 256-row tile and a few more."""
    x, w = inputs.problem(4096, 10240, 8192, seed=0, act="outlier")
    rows = np.unique(np.concatenate([np.arange(131, 4096, 256), [0, 1, 4095]]))
    run_f6(dev, x, w, rows=rows, want_p=False)


@pytest.mark.gpu
def test_f6_argument_checks(dev):
    x = torch.zeros((4, 256), dtype=torch.float16, device=dev)
    with pytest.raises(apex4.Apex4Error):
        apex4.quantize_f6(x, 64)
    L = apex4.lib()
    s = torch.ones((4, 1), dtype=torch.float32, device=dev)
    q = torch.zeros((64, 150), dtype=torch.uint8, device=dev)
    y = torch.empty((4, 4), dtype=torch.float16, device=dev)
    st = torch.cuda.current_stream().cuda_stream
    # K = 200 is not a multiple of 128
    assert L.apex4_gemm_w4a4_f6(apex4._ptr(q), apex4._ptr(s), apex4._ptr(q), apex4._ptr(s), 4, 4, 200,
                                apex4._ptr(y), None, None, None, 0, st) == 1
