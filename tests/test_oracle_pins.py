"""Pins for the CPU oracle against facts it does not compute itself.

Each test checks the oracle (oracle/apex4_oracle.c) against something fixed by
the format definitions, hand-worked cases, closed forms or an independent
fp64/int64 computation, chosen so that a plausible slip (a dropped term, a
wrong sign, index or scale, a transposed operand, round-half-away instead of
half-even, multiply-by-reciprocal instead of divide) fails at least one.
"""
import os

import numpy as np
import pytest

from w4a4_group_quantized_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- helpers


def _codes_np(packed, K):
    """Independent numpy decode of two's-complement nibbles (low nibble = even k)."""
    lo = (packed & 0x0F).astype(np.int16)
    hi = (packed >> 4).astype(np.int16)
    c = np.empty((packed.shape[0], K), dtype=np.int16)
    c[:, 0::2] = lo
    c[:, 1::2] = hi
    c[c >= 8] -= 16
    return c.astype(np.int64)


def _read_quant_cases():
    cases, cur = [], {}
    with open(os.path.join(GOLDEN, "quant_cases.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = line.split(":", 1)
            cur[key] = val.split()
            if key == "codes":
                cases.append(cur)
                cur = {}
    return cases


# ---------------------------------------------------------------- fp16 format


def test_f16_to_f32_all_bit_patterns(oracle_mod):
    """Every binary16 pattern decodes as numpy's IEEE binary16 does."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = np.array([oracle_mod.f16_to_f32(int(b)) for b in bits], dtype=np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f32_to_f16_matches_ieee_rne(oracle_mod):
    """fp32 -> fp16 rounding agrees with numpy on ties, subnormals and overflow."""
    rng = np.random.default_rng(5)
    h = np.arange(0, 0x7C00, dtype=np.uint16)
    v = h.view(np.float16).astype(np.float32)
    nxt = (h + 1).view(np.float16).astype(np.float32)
    mids = ((v.astype(np.float64) + nxt.astype(np.float64)) / 2).astype(np.float32)  # exact ties
    vals = np.concatenate([
        v, mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(np.inf)),
        rng.standard_normal(20000).astype(np.float32) * np.float32(100),
        np.float32([65504, 65519.99, 65520, 65536, 1e9, 2.0**-25, 2.0**-26, 3 * 2.0**-26,
                    2.0**-24, 1e-30]),
    ])
    vals = np.concatenate([vals, -vals])
    got = np.array([oracle_mod.f32_to_f16(float(x)) for x in vals], dtype=np.uint16)
    with np.errstate(over="ignore"):
        ref = vals.astype(np.float16).view(np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(vals[i]), hex(got[i]), hex(ref[i])) for i in bad[:5]]


# ---------------------------------------------------------------- quantization


def test_quantize_hand_cases(oracle_mod):
    """Hand-worked tie, zero-group and scale cases (tests/golden/quant_cases.txt)."""
    cases = _read_quant_cases()
    assert len(cases) >= 6
    for c in cases:
        x = np.array([float(v) for v in c["x"]], dtype=np.float16)[None, :]
        g = x.shape[1]
        q, s = oracle_mod.quantize(x, g)
        assert s.shape == (1, 1)
        assert s[0, 0].view(np.uint32) == int(c["scale"][0], 16), c
        got = _codes_np(q, g)[0]
        assert got.tolist() == [int(v) for v in c["codes"]], c


def test_pack_bytes_fixture(oracle_mod):
    """Byte layout (tests/golden/pack_cases.txt): decode, and encode via quantize."""
    rows = []
    with open(os.path.join(GOLDEN, "pack_cases.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                a, b, h = line.split()
                rows.append((int(a), int(b), int(h, 16)))
    packed = np.array([[r[2] for r in rows]], dtype=np.uint8)
    K = 2 * len(rows)
    codes = oracle_mod.codes(packed, K)[0]
    assert codes[0::2].tolist() == [r[0] for r in rows]
    assert codes[1::2].tolist() == [r[1] for r in rows]
    # encode: with an absmax-7 group the codes equal the inputs, so quantize must
    # emit the fixture byte for every pair the quantizer can produce (not -8)
    for a, b, h in rows:
        if -8 in (a, b):
            continue
        x = np.array([[a, b, 7, 0]], dtype=np.float16)
        q, s = oracle_mod.quantize(x, 4)
        assert s[0, 0] == 1.0
        assert q[0, 0] == h, (a, b, hex(q[0, 0]), hex(h))


@pytest.mark.parametrize("kind", inputs.ACT_KINDS)
@pytest.mark.parametrize("g", [32, 128, 256])
def test_quantize_invariants(oracle_mod, kind, g):
    rng = np.random.default_rng(11)
    x = inputs.activations(rng, 24, 1024, kind, seed=11)
    x[3, :g] = 0  # one all-zero group
    q, s = oracle_mod.quantize(x, g)
    c = _codes_np(q, 1024)
    xf = x.astype(np.float64)
    R, K = x.shape
    G = K // g
    xg = xf.reshape(R, G, g)
    cg = c.reshape(R, G, g)
    amax = np.abs(xg).max(axis=2)
    # the scale is the fp32 quotient absmax / 7
    assert np.array_equal(s, (amax.astype(np.float32) / np.float32(7)))
    # codes stay within [-7, 7]: the clamp never bites for finite input
    assert np.abs(c).max() <= 7
    # the absmax element of every nonzero group maps to +-7
    nz = amax > 0
    idx = np.abs(xg).argmax(axis=2)
    top = np.take_along_axis(cg, idx[..., None], axis=2)[..., 0]
    assert np.all(np.abs(top[nz]) == 7)
    # zero group -> scale 0, codes 0
    assert s[3, 0] == 0 and np.all(cg[3, 0] == 0)
    # reconstruction error <= s/2 plus the fp32 quotient's rounding slack
    sd = s.astype(np.float64)[..., None]
    err = np.abs(xg - cg * sd)
    assert np.all(err <= sd * (0.5 + 2.0**-21) + 0.0)
    # away from ties, the code is the fp64 nearest integer of x/s
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(sd > 0, xg / sd, 0.0)
    far = np.abs(np.abs(t - np.floor(t)) - 0.5) > 1e-5
    assert np.array_equal(cg[far], np.rint(t[far]).astype(np.int64))


def test_quantize_power_of_two_invariance(oracle_mod):
    """x * 2^e leaves the codes unchanged and multiplies the scales by exactly 2^e."""
    rng = np.random.default_rng(3)
    x = inputs.activations(rng, 8, 512, "normal", seed=3)
    q0, s0 = oracle_mod.quantize(x, 128)
    for e in (1, 2, 4):   # upward only: downward scaling can land in fp16 subnormals
        xe = (x.astype(np.float32) * np.float32(2.0**e)).astype(np.float16)
        assert np.array_equal(xe.astype(np.float32), x.astype(np.float32) * np.float32(2.0**e))
        q1, s1 = oracle_mod.quantize(xe, 128)
        assert np.array_equal(q1, q0)
        assert np.array_equal(s1, s0 * np.float32(2.0**e))


def test_quantize_rejects_nonfinite(oracle_mod):
    x = np.zeros((2, 64), dtype=np.float16)
    x[1, 5] = np.inf
    with pytest.raises(oracle_mod.OracleError):
        oracle_mod.quantize(x, 32)
    x[1, 5] = np.nan
    with pytest.raises(oracle_mod.OracleError):
        oracle_mod.quantize(x, 32)


# ---------------------------------------------------------------- GEMM


@pytest.mark.parametrize("g", [32, 64, 128, 256, 1024])
def test_gemm_unit_scales_is_integer_matmul(oracle_mod, g):
    """All scales 1: Y equals the int64 matmul exactly, P the int64 group sums."""
    M, N, K = 9, 13, 1024
    qa, _ = inputs.random_packed(M, K, 1, seed=1)
    qw, _ = inputs.random_packed(N, K, 1, seed=2)
    sa = np.ones((M, K // g), np.float32)
    sw = np.ones((N, K // g), np.float32)
    y16, y32, p = oracle_mod.gemm(qa, sa, g, qw, sw, g, K, want_p=True)
    ca, cw = _codes_np(qa, K), _codes_np(qw, K)
    assert (ca == -8).any() and (cw == -8).any()
    ref = ca @ cw.T
    assert np.abs(ref).max() < 2**24
    assert np.array_equal(y32.astype(np.int64), ref)
    assert np.array_equal(y32, ref.astype(np.float32))
    G = K // g
    pref = np.einsum("mgk,ngk->mng", ca.reshape(M, G, g), cw.reshape(N, G, g))
    assert np.array_equal(p.astype(np.int64), pref)
    assert np.array_equal(y16, ref.astype(np.float32).astype(np.float16))


def test_gemm_per_channel_closed_form(oracle_mod):
    """g = K (one group): Y32 = fl32(fl32(s_a*s_w) * P) bit for bit."""
    M, N, K = 7, 11, 512
    qa, sa = inputs.random_packed(M, K, 1, seed=4, scale_lo=1e-3, scale_hi=1.0)
    qw, sw = inputs.random_packed(N, K, 1, seed=5, scale_lo=1e-3, scale_hi=1.0)
    _, y32, _ = oracle_mod.gemm(qa, sa, K, qw, sw, K, K)
    P = (_codes_np(qa, K) @ _codes_np(qw, K).T).astype(np.float32)
    S = sa[:, 0][:, None] * sw[:, 0][None, :]          # fp32 products
    assert S.dtype == np.float32
    ref = S * P                                        # fp32 products
    assert np.array_equal(y32.view(np.uint32), ref.view(np.uint32))


def _fp64_reference(qa, sa, ga, qw, sw, gw, K):
    """Dequantize-then-matmul in fp64, plus the absolute-value sums the error bound needs."""
    ca, cw = _codes_np(qa, K).astype(np.float64), _codes_np(qw, K).astype(np.float64)
    da = ca * np.repeat(sa.astype(np.float64), ga, axis=1)
    dw = cw * np.repeat(sw.astype(np.float64), gw, axis=1)
    y64 = da @ dw.T
    gs = min(ga, gw)
    G = K // gs
    M, N = ca.shape[0], cw.shape[0]
    # sum_j |S_j P_j| with S_j, P_j exact
    Pj = np.einsum("mgk,ngk->mng", ca.reshape(M, G, gs), cw.reshape(N, G, gs))
    saj = np.repeat(sa.astype(np.float64), ga // gs, axis=1)
    swj = np.repeat(sw.astype(np.float64), gw // gs, axis=1)
    absterm = np.einsum("mg,ng,mng->mn", saj, swj, np.abs(Pj))
    absprod = np.abs(da) @ np.abs(dw).T
    return y64, absterm, absprod, G


@pytest.mark.parametrize("ga,gw", [(32, 32), (64, 64), (128, 128), (256, 256), (128, 1024),
                                   (32, 1024), (1024, 1024)])
def test_gemm_fp64_bruteforce_bound(oracle_mod, ga, gw):
    """|Y32 - Y64| within the sequential-fp32 bound (G+2)u*sum|S_j P_j| + fp64 slack."""
    M, N, K = 12, 10, 1024
    qa, sa = inputs.random_packed(M, K, K // ga, seed=6, scale_lo=1e-3, scale_hi=1e-1)
    qw, sw = inputs.random_packed(N, K, K // gw, seed=7, scale_lo=1e-3, scale_hi=1e-1)
    y16, y32, _ = oracle_mod.gemm(qa, sa, ga, qw, sw, gw, K)
    y64, absterm, absprod, G = _fp64_reference(qa, sa, ga, qw, sw, gw, K)
    u = 2.0**-24
    bound = (G + 2) * u * absterm * 1.0001 + (K + 2) * 2.0**-53 * absprod
    err = np.abs(y32.astype(np.float64) - y64)
    assert np.all(err <= bound), float((err / np.maximum(bound, 1e-300)).max())
    # and the bound is tight enough to mean something: relative error ~1e-6 or better
    assert err.max() <= 1e-5 * np.abs(y64).max()
    assert np.array_equal(y16, y32.astype(np.float16))


def test_gemm_bruteforce_catches_swapped_scales(oracle_mod):
    """Sanity of the pin itself: swapping the two scale tensors' roles is detected."""
    M, N, K, g = 6, 6, 512, 128
    qa, sa = inputs.random_packed(M, K, K // g, seed=8)
    qw, sw = inputs.random_packed(N, K, K // g, seed=9)
    _, y32, _ = oracle_mod.gemm(qa, sa, g, qw, sw, g, K)
    y64, _, _, _ = _fp64_reference(qa, sa, g, qw, sw, g, K)
    wrong, _, _, _ = _fp64_reference(qa, sw[:M], g, qw, sa[:N], g, K)
    assert np.abs(y32 - y64).max() < 1e-5 * np.abs(y64).max()
    assert np.abs(wrong - y64).max() > 1e-3 * np.abs(y64).max()


def test_gemm_from_quantized_fp_inputs(oracle_mod):
    """End to end on synthetic fp16 X and W: Y tracks X @ W^T within INT4 error."""
    x, w = inputs.problem(16, 64, 1024, seed=0, act="normal")
    qa, sa = oracle_mod.quantize(x, 128)
    qw, sw = oracle_mod.quantize(w, 128)
    y16, y32, _ = oracle_mod.gemm(qa, sa, 128, qw, sw, 128, 1024)
    y64, _, _, _ = _fp64_reference(qa, sa, 128, qw, sw, 128, 1024)
    assert np.abs(y32 - y64).max() <= 1e-5 * np.abs(y64).max()
    yfp = x.astype(np.float64) @ w.astype(np.float64).T
    rel = np.linalg.norm(y32 - yfp) / np.linalg.norm(yfp)
    assert 0.01 < rel < 0.25, rel   # 4-bit noise: clearly nonzero, clearly bounded


def test_gemm_power_of_two_invariance(oracle_mod):
    """Scaling X by 2^e scales Y32 by exactly 2^e (no over/underflow here)."""
    x, w = inputs.problem(8, 24, 512, seed=2, act="outlier")
    qw, sw = oracle_mod.quantize(w, 128)
    qa, sa = oracle_mod.quantize(x, 128)
    _, y0, _ = oracle_mod.gemm(qa, sa, 128, qw, sw, 128, 512)
    xe = (x.astype(np.float32) * np.float32(8)).astype(np.float16)
    qa2, sa2 = oracle_mod.quantize(xe, 128)
    _, y1, _ = oracle_mod.gemm(qa2, sa2, 128, qw, sw, 128, 512)
    assert np.array_equal(y1, y0 * np.float32(8))


def test_gemm_rejects_bad_args(oracle_mod):
    qa = np.zeros((2, 64), np.uint8)
    s = np.ones((2, 1), np.float32)
    with pytest.raises(oracle_mod.OracleError):
        oracle_mod.gemm(qa, s, 96, qa, s, 96, 128)       # 128 % 96 != 0
    bad = s.copy()
    bad[0, 0] = np.nan
    with pytest.raises(oracle_mod.OracleError):
        oracle_mod.gemm(qa, bad, 128, qa, s, 128, 128)
