"""CPU-side checks of the C ABI (include/apex4.h, include/apex4_probe.h): the
library loads, exports every declared symbol, and rejects bad arguments on the
host with the documented status codes.  No call here reaches the GPU: every call fails a
host-side check, which runs before any HIP call."""
import ctypes
import glob
import os
import re
import subprocess

import pytest

from w4a4_group_quantized_amd import apex4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))

OK, INVALID, UNSUPPORTED, ALIGN, WORKSPACE, HIP = 0, 1, 2, 3, 4, 5
A16 = 0x10000          # fake, 16-byte aligned device addresses: never dereferenced
A16b = 0x20000
MIS = 0x10001          # misaligned


def declared_functions():
    names = set()
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(apex4_\w+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(apex4.LIB_PATH):
        pytest.skip("libapex4.so not built (run __graft_entry__.build())")
    return apex4.lib()


def test_header_and_binding_agree():
    assert declared_functions() == sorted(apex4.SIGNATURES)


def test_library_exports_every_declared_symbol(L):
    out = subprocess.run(["nm", "-D", "--defined-only", apex4.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (apex4_\w+)", out))
    for name in declared_functions():
        assert name in exported, name
        assert getattr(L, name) is not None


def test_status_strings(L):
    for code in range(6):
        s = L.apex4_status_string(code)
        assert s and s.decode() != "unknown status"
    assert L.apex4_status_string(99).decode() == "unknown status"


def test_workspace_size_is_zero(L):
    assert L.apex4_gemm_workspace_size(2048, 12288, 4096, 128, 128) == 0


@pytest.mark.parametrize("fn", ["apex4_quantize_act", "apex4_pack_weight"])
def test_quantize_validation(L, fn):
    f = getattr(L, fn)
    # K not a multiple of 8
    assert f(A16, 4, 100, 4, A16b, A16b, None) == INVALID
    # group does not divide K
    assert f(A16, 4, 1024, 96, A16b, A16b, None) == INVALID
    # group not in {32,64,128,256,K}
    assert f(A16, 4, 1024, 16, A16b, A16b, None) == UNSUPPORTED
    assert f(A16, 4, 1024, 512, A16b, A16b, None) == UNSUPPORTED
    # negative rows, zero K
    assert f(A16, -1, 1024, 128, A16b, A16b, None) == INVALID
    assert f(A16, 4, 0, 128, A16b, A16b, None) == INVALID
    # null pointers
    assert f(None, 4, 1024, 128, A16b, A16b, None) == INVALID
    assert f(A16, 4, 1024, 128, None, A16b, None) == INVALID
    # misaligned input
    assert f(MIS, 4, 1024, 128, A16b, A16b, None) == ALIGN
    assert f(A16, 4, 1024, 128, A16b, A16b + 2, None) == ALIGN
    # empty input: a successful no-op that touches nothing
    assert f(None, 0, 1024, 128, None, None, None) == OK


def _gemm(L, qa=A16, sa=A16b, ga=128, qw=A16, sw=A16b, gw=128, M=16, N=16, K=1024,
          y16=A16b, y32=None, ps=None, ws=None, wsb=0):
    return L.apex4_gemm_w4a4(qa, sa, ga, qw, sw, gw, M, N, K, y16, y32, ps, ws, wsb, None)


def test_gemm_validation(L):
    assert _gemm(L, K=1000) == INVALID                 # K % 128
    assert _gemm(L, K=0) == INVALID
    assert _gemm(L, M=-1) == INVALID
    assert _gemm(L, ga=96, gw=96) == INVALID           # does not divide K
    assert _gemm(L, ga=512, gw=512) == UNSUPPORTED     # not in {32..256, K}
    assert _gemm(L, ga=128, gw=64) == UNSUPPORTED      # neither equal nor mixed
    assert _gemm(L, ga=1024, gw=128) == UNSUPPORTED    # converse of mixed mode
    assert _gemm(L, qa=None) == INVALID
    assert _gemm(L, y16=None) == INVALID
    assert _gemm(L, qa=MIS) == ALIGN
    assert _gemm(L, qw=A16 + 8) == ALIGN
    assert _gemm(L, y16=A16b + 1) == ALIGN
    assert _gemm(L, y32=A16b + 2) == ALIGN
    # psum too large for 32-bit indexing
    assert _gemm(L, M=65536, N=65536, ps=A16b) == INVALID
    # empty shapes are successful no-ops
    assert _gemm(L, M=0, qa=None, sa=None, y16=None) == OK
    assert _gemm(L, N=0, qw=None, sw=None, y16=None) == OK


def test_linear_workspace_layout(L):
    """apex4_linear_workspace_size: 0 for the fused decode shapes; otherwise
    the activation codes, then their scales (each 256-byte aligned), then the
    GEMM's own workspace.  (Host arithmetic; the ping-pong split's share
    depends on the device's compute units, so it is taken from
    apex4_gemm_workspace_size in the same process.)"""
    assert L.apex4_linear_workspace_size(1, 28672, 8192, 128, 128) == 0
    assert L.apex4_linear_workspace_size(2, 28672, 8192, 256, 256) == 0

    def a256(b):
        return (b + 255) // 256 * 256
    for M, N, K, ga, gw in [(1, 8192, 28672, 128, 128), (2, 512, 1024, 1024, 1024), (3, 1000, 1024, 64, 64),
                            (40, 8192, 28672, 128, 128), (300, 1000, 1024, 128, 1024)]:
        expect = a256(M * K // 2) + a256(M * (K // ga) * 4) + L.apex4_gemm_workspace_size(M, N, K, ga, gw)
        assert L.apex4_linear_workspace_size(M, N, K, ga, gw) == expect, (M, N, K, ga, gw)
    # the K-outer kernel's two K halves (17-64 rows, at most 2 column blocks per workgroup)
    assert L.apex4_gemm_workspace_size(40, 8192, 28672, 128, 128) == 2 * 40 * 8192 * 4
    # invalid arguments: 0 (the call itself reports them)
    assert L.apex4_linear_workspace_size(1, 64, 200, 128, 128) == 0
    assert L.apex4_linear_workspace_size(0, 64, 256, 128, 128) == 0


def _linear(L, x=A16, ga=128, qw=A16, sw=A16b, gw=128, M=1, N=16, K=1024, y16=A16b, y32=None, ws=None, wsb=0):
    return L.apex4_linear_w4a4(x, ga, qw, sw, gw, M, N, K, y16, y32, ws, wsb, None)


def test_linear_validation(L):
    assert _linear(L, K=1000) == INVALID               # K % 128
    assert _linear(L, ga=96, gw=96) == INVALID         # does not divide K
    assert _linear(L, ga=512, gw=512) == UNSUPPORTED   # not in {32..256, K}
    assert _linear(L, ga=128, gw=64) == UNSUPPORTED    # neither equal nor mixed
    assert _linear(L, M=40, N=8192, K=28672) == WORKSPACE     # needs the codes, scales and K halves
    assert _linear(L, M=40, N=8192, K=28672, ws=A16, wsb=1000) == WORKSPACE
    assert _linear(L, x=None) == INVALID
    assert _linear(L, y16=None) == INVALID
    assert _linear(L, x=MIS) == ALIGN
    assert _linear(L, y32=A16b + 2) == ALIGN
    assert _linear(L, M=3, ws=A16 + 16, wsb=1 << 20) == ALIGN   # workspace not 256-byte aligned
    # empty shapes are successful no-ops
    assert _linear(L, M=0, x=None, y16=None) == OK
    assert _linear(L, N=0, qw=None, sw=None, y16=None) == OK


def test_probe_validation(L):
    """The probes check their arguments on the host (nothing is launched)."""
    d = ctypes.c_double(0.0)
    assert L.apex4_probe_mfma_i8(0, A16, ctypes.byref(d), None) == INVALID
    assert L.apex4_probe_mfma_i8(10, None, ctypes.byref(d), None) == INVALID
    assert L.apex4_probe_mfma_i8(10, MIS, ctypes.byref(d), None) == ALIGN
    assert L.apex4_probe_mfma_f6(0, A16, ctypes.byref(d), None) == INVALID
    assert L.apex4_probe_mfma_f6(10, None, ctypes.byref(d), None) == INVALID
    assert L.apex4_probe_mfma_f6(10, MIS, ctypes.byref(d), None) == ALIGN
    assert L.apex4_probe_valu_f32(0, A16, ctypes.byref(d), None) == INVALID
    assert L.apex4_probe_valu_f32(10, A16, None, None) == INVALID
    assert L.apex4_probe_lds_read(0, A16, ctypes.byref(d), None) == INVALID
    assert L.apex4_probe_lds_read(1 << 31, A16, ctypes.byref(d), None) == INVALID
    assert L.apex4_probe_lds_read(10, MIS, ctypes.byref(d), None) == ALIGN
    assert L.apex4_probe_hbm_read(A16, 4095, A16b, ctypes.byref(d), None) == INVALID
    assert L.apex4_probe_hbm_read(A16, 0, A16b, ctypes.byref(d), None) == INVALID
    assert L.apex4_probe_hbm_read(None, 4096, A16b, ctypes.byref(d), None) == INVALID
    assert L.apex4_probe_hbm_read(MIS, 4096, A16b, ctypes.byref(d), None) == ALIGN


def test_per_channel_int32_limit(L):
    """One group over all of K keeps 256 * P in one int32: K < 2^17.  The
    refusal comes before the pointer checks, so a NULL y16 tells the two
    apart: UNSUPPORTED at K = 2^17, the next check (INVALID) just below."""
    big, ok = 1 << 17, (1 << 17) - 128
    assert _gemm(L, ga=big, gw=big, K=big) == UNSUPPORTED
    assert _gemm(L, ga=ok, gw=ok, K=ok, y16=None) == INVALID
    # groups of 128 and mixed mode sum at most one group of 128 per int32
    assert _gemm(L, ga=128, gw=128, K=big, y16=None) == INVALID
    assert _gemm(L, ga=128, gw=big, K=big, y16=None) == INVALID
    assert _linear(L, ga=big, gw=big, K=big) == UNSUPPORTED
    assert _linear(L, ga=ok, gw=ok, K=ok) == WORKSPACE      # (its next check: the codes need a workspace)
    assert L.apex4_gemm_workspace_size(4096, 4096, big, big, big) == 0
    assert L.apex4_linear_workspace_size(4096, 4096, big, big, big) == 0


def _gemm_dbg(L, M=16, N=16, K=1024, ga=128, row0=0, step=1, rows=16, ps=A16b, y16=A16b):
    return L.apex4_gemm_w4a4_debug(A16, A16b, ga, A16, A16b, ga, M, N, K, y16, None, row0, step, rows, ps,
                                   None, 0, None)


def test_gemm_debug_rows_validation(L):
    """apex4_gemm_w4a4_debug: the kept rows must lie inside Y and their sums fit
    32-bit indexing; otherwise INVALID before anything is launched.  (Valid
    row selections pass on to the next check: a NULL y16 gives INVALID there
    too, so those are told apart by the other arguments being valid.)"""
    assert _gemm_dbg(L, step=0) == INVALID
    assert _gemm_dbg(L, row0=-1) == INVALID
    assert _gemm_dbg(L, rows=-1) == INVALID
    assert _gemm_dbg(L, row0=15, step=1, rows=2) == INVALID          # row 16 of 16
    assert _gemm_dbg(L, M=300, row0=44, step=256, rows=2) == INVALID  # row 300 of 300
    assert _gemm_dbg(L, ps=None) == INVALID                           # sums asked, no buffer
    assert _gemm_dbg(L, M=1 << 20, N=1 << 20, rows=4096, step=256) == INVALID   # 2^32 sums
    assert _gemm_dbg(L, ps=A16b + 2) == ALIGN
    # the same call with every argument valid but y16 is stopped at y16
    assert _gemm_dbg(L, M=300, row0=43, step=256, rows=2, y16=None) == INVALID
    # no rows kept: no sums buffer needed; empty shapes stay no-ops
    assert _gemm_dbg(L, rows=0, ps=None, y16=A16b + 1) == ALIGN
    assert L.apex4_gemm_w4a4_debug(None, None, 128, A16, A16b, 128, 0, 16, 1024, None, None, 0, 1, 0, None,
                                   None, 0, None) == OK


class _FakeGpuTensor:
    """Just enough of a torch tensor for the binding's argument checks (which
    run before anything is allocated or launched)."""

    def __init__(self, shape, dtype, contiguous=True, device="cuda:0"):
        import torch
        self.shape = tuple(shape)
        self.dtype = dtype
        self._contig = contiguous
        self.device = torch.device(device)
        self.is_cuda = True

    def is_contiguous(self):
        return self._contig


def test_binding_refuses_mismatched_tensors():
    """apex4.gemm / quantize_act check shapes, dtypes, contiguity and device
    against (M, N, K, groups) before calling the library: a mismatch would
    otherwise make a kernel read or write out of bounds."""
    torch = pytest.importorskip("torch")
    T = _FakeGpuTensor
    M, N, K = 8, 16, 256
    qa, sa = T((M, K // 2), torch.uint8), T((M, K // 128), torch.float32)
    qw, sw = T((N, K // 2), torch.uint8), T((N, K // 128), torch.float32)
    bad = [
        dict(qa=T((M, K // 4), torch.uint8)),                       # K/2 columns expected
        dict(sa=T((M, K // 64), torch.float32)),                    # K/ga scale columns
        dict(sw=T((N + 1, K // 128), torch.float32)),               # N rows
        dict(sa=T((M, K // 128), torch.float16)),                   # fp32 scales
        dict(qw=T((N, K // 2), torch.uint8, contiguous=False)),
        dict(qw=T((N, K // 2), torch.uint8, device="cuda:1")),      # another device
        dict(y16=T((M, N - 1), torch.float16)),
        dict(y16=T((M, N), torch.float16, contiguous=False)),
        dict(y32=T((M, N), torch.float16)),
    ]
    for b in bad:
        args = dict(qa=qa, sa=sa, qw=qw, sw=sw, y16=None, y32=None)
        args.update(b)
        with pytest.raises(ValueError):
            apex4.gemm(args["qa"], args["sa"], 128, args["qw"], args["sw"], 128, K,
                       y16=args["y16"], y32=args["y32"])
    # an explicit K that disagrees with the codes
    with pytest.raises(ValueError):
        apex4.gemm(qa, sa, 128, qw, sw, 128, 2 * K)
    # quantize_act into caller buffers of the wrong shape
    x = T((M, K), torch.float16)
    with pytest.raises(ValueError):
        apex4.quantize_act(x, 128, out=(T((M, K // 2), torch.uint8), T((M, 1), torch.float32)))
    with pytest.raises(ValueError):
        apex4.quantize_act(x, 128, out=(T((M, K), torch.uint8), T((M, K // 128), torch.float32)))


def test_noalloc_host_checks(L):
    """apex4_gemm_w4a4_noalloc: the checks of apex4_gemm_w4a4 on the host,
    before anything is looked up or launched; the scratch size in the header
    and in the binding agree."""
    f = L.apex4_gemm_w4a4_noalloc
    assert f(A16, A16b, 128, A16, A16b, 128, 16, 16, 1000, A16b, None, None) == INVALID     # K % 128
    assert f(A16, A16b, 96, A16, A16b, 96, 16, 16, 1024, A16b, None, None) == INVALID       # group
    assert f(A16, A16b, 512, A16, A16b, 512, 16, 16, 1024, A16b, None, None) == UNSUPPORTED
    assert f(A16, A16b, 128, A16, A16b, 128, 16, 16, 1024, None, None, None) == INVALID     # NULL y16
    assert f(MIS, A16b, 128, A16, A16b, 128, 16, 16, 1024, A16b, None, None) == ALIGN
    assert f(None, None, 128, A16, A16b, 128, 0, 16, 1024, None, None, None) == OK          # empty
    text = open(os.path.join(ROOT, "include", "apex4.h")).read()
    m = re.search(r"#define APEX4_NOALLOC_MAX_WORKSPACE \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == apex4.NOALLOC_MAX_WORKSPACE


def test_f8_group_checks(L):
    """apex4_quantize_f8 / apex4_gemm_w4a4_f8: groups of 64 and 128 only, checked on the
    host before any pointer is used (M = 0 would otherwise be a no-op)."""
    assert L.apex4_quantize_f8(A16, 4, 1024, 32, A16b, A16b, None) == UNSUPPORTED
    assert L.apex4_quantize_f8(A16, 4, 1024, 256, A16b, A16b, None) == UNSUPPORTED
    assert L.apex4_quantize_f8(A16, 4, 1024, 96, A16b, A16b, None) == INVALID     # does not divide K
    f = L.apex4_gemm_w4a4_f8
    assert f(A16, A16b, A16, A16b, 32, 0, 8, 1024, A16, None, None, None) == UNSUPPORTED
    assert f(A16, A16b, A16, A16b, 256, 0, 8, 1024, A16, None, None, None) == UNSUPPORTED
    assert f(A16, A16b, A16, A16b, 96, 0, 8, 1024, A16, None, None, None) == INVALID
    assert f(A16, A16b, A16, A16b, 0, 0, 8, 1024, A16, None, None, None) == INVALID
    assert f(A16, A16b, A16, A16b, 64, 8, 8, 1000, A16, None, None, None) == INVALID   # K % 128
    for g in (64, 128):
        assert f(A16, A16b, A16, A16b, g, 0, 8, 1024, A16, None, None, None) == OK    # no-op
        assert f(MIS, A16b, A16, A16b, g, 8, 8, 1024, A16, None, None, None) == ALIGN
