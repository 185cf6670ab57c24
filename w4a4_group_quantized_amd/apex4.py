"""Thin ctypes binding of libapex4.so (the C ABI in include/apex4.h).

Argument marshalling only: every step of the W4A4 path runs in the HIP
kernels behind the C ABI.  Tensors are torch tensors on the GPU (PyTorch is
used for device memory and streams); calls go on torch's current stream.
There is no CPU fallback: without the built library or a GPU tensor these
functions raise.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# APEX4_LIB selects another build of the same library (e.g. a tuning variant)
LIB_PATH = os.environ.get("APEX4_LIB", os.path.join(PKG, "libapex4.so"))

OK = 0
# APEX4_NOALLOC_MAX_WORKSPACE: the per-GPU scratch array of apex4_gemm_w4a4_noalloc
NOALLOC_MAX_WORKSPACE = 32 << 20
STATUS_NAMES = {0: "APEX4_OK", 1: "APEX4_ERR_INVALID_ARG", 2: "APEX4_ERR_UNSUPPORTED",
                3: "APEX4_ERR_ALIGNMENT", 4: "APEX4_ERR_WORKSPACE", 5: "APEX4_ERR_HIP"}

# name -> (restype, argtypes); mirrors include/apex4.h and include/apex4_probe.h
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
SIGNATURES = {
    "apex4_status_string": (ctypes.c_char_p, [_I32]),
    "apex4_quantize_act": (_I32, [_P, _I64, _I64, _I32, _P, _P, _P]),
    "apex4_pack_weight": (_I32, [_P, _I64, _I64, _I32, _P, _P, _P]),
    "apex4_gemm_workspace_size": (ctypes.c_size_t, [_I64, _I64, _I64, _I32, _I32]),
    "apex4_gemm_w4a4": (_I32, [_P, _P, _I32, _P, _P, _I32, _I64, _I64, _I64,
                               _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "apex4_gemm_w4a4_debug": (_I32, [_P, _P, _I32, _P, _P, _I32, _I64, _I64, _I64,
                                     _P, _P, _I64, _I64, _I64, _P, _P, ctypes.c_size_t, _P]),
    "apex4_gemm_w4a4_noalloc": (_I32, [_P, _P, _I32, _P, _P, _I32, _I64, _I64, _I64, _P, _P, _P]),
    "apex4_linear_workspace_size": (ctypes.c_size_t, [_I64, _I64, _I64, _I32, _I32]),
    "apex4_linear_w4a4": (_I32, [_P, _I32, _P, _P, _I32, _I64, _I64, _I64, _P, _P, _P, ctypes.c_size_t, _P]),
    "apex4_quantize_f8": (_I32, [_P, _I64, _I64, _I32, _P, _P, _P]),
    "apex4_gemm_w4a4_f8": (_I32, [_P, _P, _P, _P, _I32, _I64, _I64, _I64, _P, _P, _P, _P]),
    "apex4_quantize_f6": (_I32, [_P, _I64, _I64, _I32, _P, _P, _P]),
    "apex4_gemm_w4a4_f6": (_I32, [_P, _P, _P, _P, _I64, _I64, _I64, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "apex4_select_granularity": (_I32, [_I64, _I64, _I64, ctypes.c_double,
                                        ctypes.POINTER(_I32), ctypes.POINTER(_I32)]),
    "apex4_probe_mfma_i8": (_I32, [_I64, _P, ctypes.POINTER(ctypes.c_double), _P]),
    "apex4_probe_mfma_f6": (_I32, [_I64, _P, ctypes.POINTER(ctypes.c_double), _P]),
    "apex4_probe_hbm_read": (_I32, [_P, _I64, _P, ctypes.POINTER(ctypes.c_double), _P]),
    "apex4_probe_valu_f32": (_I32, [_I64, _P, ctypes.POINTER(ctypes.c_double), _P]),
    "apex4_probe_lds_read": (_I32, [_I64, _P, ctypes.POINTER(ctypes.c_double), _P]),
}

_lib = None


class Apex4Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS_NAMES.get(status, status)} "
                         f"({lib().apex4_status_string(status).decode()})")


def lib() -> ctypes.CDLL:
    """Load libapex4.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run `python -m w4a4_group_quantized_amd.build` "
                               "(or __graft_entry__.build()) first")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(fn: str, status: int) -> None:
    if status != OK:
        raise Apex4Error(fn, status)


def _stream(torch, device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _need_gpu(t, name: str, dtype=None, shape=None, device=None) -> None:
    """Refuse what the C ABI cannot check itself: a host tensor, a
    non-contiguous one, the wrong dtype, the wrong shape or another device."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (this library has no CPU path)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the call runs on {device}")


def _cols(K: int, group: int) -> int:
    """Scale columns K / group (0 for a group the library will refuse)."""
    return K // group if group > 0 else 0


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def quantize_act(x, group: int, out=None):
    """x: fp16 [M, K] GPU tensor -> (qa uint8 [M, K/2], s_a float32 [M, K/group])."""
    import torch
    _need_gpu(x, "x", torch.float16)
    M, K = x.shape
    if out is None:
        qa = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device)
        sa = torch.empty((M, _cols(K, group)), dtype=torch.float32, device=x.device)
    else:
        qa, sa = out
        _need_gpu(qa, "qa", torch.uint8, (M, K // 2), x.device)
        _need_gpu(sa, "s_a", torch.float32, (M, _cols(K, group)), x.device)
    _check("apex4_quantize_act", lib().apex4_quantize_act(
        _ptr(x), M, K, group, _ptr(qa), _ptr(sa), _stream(torch, x.device)))
    return qa, sa


def pack_weight(w, group: int):
    """w: fp16 [N, K] GPU tensor -> (qw uint8 [N, K/2], s_w float32 [N, K/group])."""
    import torch
    _need_gpu(w, "w", torch.float16)
    N, K = w.shape
    qw = torch.empty((N, K // 2), dtype=torch.uint8, device=w.device)
    sw = torch.empty((N, _cols(K, group)), dtype=torch.float32, device=w.device)
    _check("apex4_pack_weight", lib().apex4_pack_weight(
        _ptr(w), N, K, group, _ptr(qw), _ptr(sw), _stream(torch, w.device)))
    return qw, sw


def workspace_size(M: int, N: int, K: int, ga: int, gw: int) -> int:
    return int(lib().apex4_gemm_workspace_size(M, N, K, ga, gw))


def gemm(qa, sa, ga: int, qw, sw, gw: int, K: int | None = None, *, want_y32: bool = False,
         want_psum: bool = False, psum_rows: tuple | None = None, y16=None, y32=None):
    """Y = W4A4 GEMM with per-group dequantization (include/apex4.h).

    Returns y16 [M, N] fp16, or (y16, y32, psum) when want_y32/want_psum is set
    (entries not asked for are None).  psum_rows = (row0, step, count) keeps
    the group sums of rows row0 + i * step only (apex4_gemm_w4a4_debug):
    psum is then [count, N, G].
    """
    import torch
    M, N = qa.shape[0], qw.shape[0]
    K = 2 * qa.shape[1] if K is None else K
    dev = qa.device
    _need_gpu(qa, "qa", torch.uint8, (M, K // 2), dev)
    _need_gpu(qw, "qw", torch.uint8, (N, K // 2), dev)
    _need_gpu(sa, "s_a", torch.float32, (M, _cols(K, ga)), dev)
    _need_gpu(sw, "s_w", torch.float32, (N, _cols(K, gw)), dev)
    # caller buffers are checked before anything is allocated
    if y16 is not None:
        _need_gpu(y16, "y16", torch.float16, (M, N), dev)
    if y32 is not None:
        _need_gpu(y32, "y32", torch.float32, (M, N), dev)
    if y16 is None:
        y16 = torch.empty((M, N), dtype=torch.float16, device=dev)
    if want_y32 and y32 is None:
        y32 = torch.empty((M, N), dtype=torch.float32, device=dev)
    psum = None
    G = _cols(K, min(ga, gw))
    row0, step, count = psum_rows if psum_rows is not None else (0, 1, M)
    if want_psum:
        psum = torch.empty((count, N, G), dtype=torch.int32, device=dev)
    ws_bytes = workspace_size(M, N, K, ga, gw)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    if psum_rows is None:
        _check("apex4_gemm_w4a4", lib().apex4_gemm_w4a4(
            _ptr(qa), _ptr(sa), ga, _ptr(qw), _ptr(sw), gw, M, N, K,
            _ptr(y16), _ptr(y32), _ptr(psum), _ptr(ws), ws_bytes, _stream(torch, dev)))
    else:
        _check("apex4_gemm_w4a4_debug", lib().apex4_gemm_w4a4_debug(
            _ptr(qa), _ptr(sa), ga, _ptr(qw), _ptr(sw), gw, M, N, K,
            _ptr(y16), _ptr(y32), row0, step, count if want_psum else 0, _ptr(psum),
            _ptr(ws), ws_bytes, _stream(torch, dev)))
    if want_y32 or want_psum:
        return y16, y32, psum
    return y16


def gemm_noalloc(qa, sa, ga: int, qw, sw, gw: int, K: int | None = None, *, y16, y32=None):
    """apex4_gemm_w4a4_noalloc: the GEMM into caller-provided outputs with no
    workspace and no allocation (y16, and y32 when given, are written)."""
    import torch
    M, N = qa.shape[0], qw.shape[0]
    K = 2 * qa.shape[1] if K is None else K
    dev = qa.device
    _need_gpu(qa, "qa", torch.uint8, (M, K // 2), dev)
    _need_gpu(qw, "qw", torch.uint8, (N, K // 2), dev)
    _need_gpu(sa, "s_a", torch.float32, (M, _cols(K, ga)), dev)
    _need_gpu(sw, "s_w", torch.float32, (N, _cols(K, gw)), dev)
    _need_gpu(y16, "y16", torch.float16, (M, N), dev)
    if y32 is not None:
        _need_gpu(y32, "y32", torch.float32, (M, N), dev)
    _check("apex4_gemm_w4a4_noalloc", lib().apex4_gemm_w4a4_noalloc(
        _ptr(qa), _ptr(sa), ga, _ptr(qw), _ptr(sw), gw, M, N, K, _ptr(y16), _ptr(y32), _stream(torch, dev)))
    return y16


def linear_workspace_size(M: int, N: int, K: int, ga: int, gw: int) -> int:
    return int(lib().apex4_linear_workspace_size(M, N, K, ga, gw))


def linear(x, ga: int, qw, sw, gw: int, *, want_y32: bool = False, y16=None, y32=None, workspace=None):
    """apex4_linear_w4a4: Y of quantize_act(x) then gemm in one call (the decode
    kernel quantizes 1-2 rows itself).  x: fp16 [M, K]; returns y16, or
    (y16, y32) with want_y32.  `workspace`: a uint8 GPU tensor of at least
    linear_workspace_size() bytes (allocated here when None)."""
    import torch
    _need_gpu(x, "x", torch.float16)
    M, K = x.shape
    N = qw.shape[0]
    dev = x.device
    _need_gpu(qw, "qw", torch.uint8, (N, K // 2), dev)
    _need_gpu(sw, "s_w", torch.float32, (N, _cols(K, gw)), dev)
    # caller buffers are checked before anything is allocated
    if y16 is not None:
        _need_gpu(y16, "y16", torch.float16, (M, N), dev)
    if y32 is not None:
        _need_gpu(y32, "y32", torch.float32, (M, N), dev)
    if y16 is None:
        y16 = torch.empty((M, N), dtype=torch.float16, device=dev)
    if want_y32 and y32 is None:
        y32 = torch.empty((M, N), dtype=torch.float32, device=dev)
    need = linear_workspace_size(M, N, K, ga, gw)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace is not None:
        _need_gpu(workspace, "workspace", torch.uint8, None, dev)
    nbytes = 0 if workspace is None else workspace.numel()
    _check("apex4_linear_w4a4", lib().apex4_linear_w4a4(
        _ptr(x), ga, _ptr(qw), _ptr(sw), gw, M, N, K, _ptr(y16), _ptr(y32), _ptr(workspace), nbytes,
        _stream(torch, dev)))
    return (y16, y32) if want_y32 else y16


def quantize_f8(x, group: int = 128, out=None):
    """x: fp16 [rows, K] GPU tensor -> (q8 uint8 [rows, K] E4M3 codes, s float32 [rows, K/group])
    (apex4_quantize_f8: the rule of quantize_act / pack_weight, one byte per code; groups of 64
    or 128)."""
    import torch
    _need_gpu(x, "x", torch.float16)
    rows, K = x.shape
    if out is None:
        q8 = torch.empty((rows, K), dtype=torch.uint8, device=x.device)
        s = torch.empty((rows, _cols(K, group)), dtype=torch.float32, device=x.device)
    else:
        q8, s = out
        _need_gpu(q8, "q8", torch.uint8, (rows, K), x.device)
        _need_gpu(s, "s", torch.float32, (rows, _cols(K, group)), x.device)
    _check("apex4_quantize_f8", lib().apex4_quantize_f8(
        _ptr(x), rows, K, group, _ptr(q8), _ptr(s), _stream(torch, x.device)))
    return q8, s


def gemm_f8(qa8, sa, qw8, sw, group: int | None = None, *, want_y32: bool = False, want_psum: bool = False,
            y16=None, y32=None):
    """apex4_gemm_w4a4_f8: the W4A4 GEMM (groups of 64 or 128 on both operands; None: K / the
    scale columns) on E4M3-coded operands.  Returns y16, or (y16, y32, psum) when
    want_y32/want_psum is set."""
    import torch
    M, K = qa8.shape
    N = qw8.shape[0]
    dev = qa8.device
    if group is None:
        group = K // sa.shape[1] if sa.dim() == 2 and sa.shape[1] > 0 else 0
    _need_gpu(qa8, "qa8", torch.uint8, (M, K), dev)
    _need_gpu(qw8, "qw8", torch.uint8, (N, K), dev)
    _need_gpu(sa, "s_a", torch.float32, (M, _cols(K, group)), dev)
    _need_gpu(sw, "s_w", torch.float32, (N, _cols(K, group)), dev)
    # caller buffers are checked before anything is allocated
    if y16 is not None:
        _need_gpu(y16, "y16", torch.float16, (M, N), dev)
    if y32 is not None:
        _need_gpu(y32, "y32", torch.float32, (M, N), dev)
    if y16 is None:
        y16 = torch.empty((M, N), dtype=torch.float16, device=dev)
    if want_y32 and y32 is None:
        y32 = torch.empty((M, N), dtype=torch.float32, device=dev)
    psum = torch.empty((M, N, _cols(K, group)), dtype=torch.int32, device=dev) if want_psum else None
    _check("apex4_gemm_w4a4_f8", lib().apex4_gemm_w4a4_f8(
        _ptr(qa8), _ptr(sa), _ptr(qw8), _ptr(sw), group, M, N, K, _ptr(y16), _ptr(y32), _ptr(psum),
        _stream(torch, dev)))
    if want_y32 or want_psum:
        return y16, y32, psum
    return y16


def f6_rows(rows: int) -> int:
    """Rows of an FP6-coded operand buffer: whole blocks of 64 (apex4_quantize_f6's tiled layout)."""
    return (rows + 63) // 64 * 64


def quantize_f6(x, group: int = 128, out=None):
    """x: fp16 [rows, K] GPU tensor -> (q6 uint8 [f6_rows(rows), 3K/4] E2M3 codes in the tiled
    layout of apex4_quantize_f6, s float32 [rows, K/group])."""
    import torch
    _need_gpu(x, "x", torch.float16)
    rows, K = x.shape
    if out is None:
        q6 = torch.empty((f6_rows(rows), K * 3 // 4), dtype=torch.uint8, device=x.device)
        s = torch.empty((rows, _cols(K, group)), dtype=torch.float32, device=x.device)
    else:
        q6, s = out
        _need_gpu(q6, "q6", torch.uint8, (f6_rows(rows), K * 3 // 4), x.device)
        _need_gpu(s, "s", torch.float32, (rows, _cols(K, group)), x.device)
    _check("apex4_quantize_f6", lib().apex4_quantize_f6(
        _ptr(x), rows, K, group, _ptr(q6), _ptr(s), _stream(torch, x.device)))
    return q6, s


def gemm_f6(qa6, sa, qw6, sw, *, want_y32: bool = False, want_psum: bool = False, y16=None, y32=None):
    """apex4_gemm_w4a4_f6: the W4A4 GEMM (groups of 128) on FP6-coded operands (tiled layout);
    M, N and K come from the scales.  Returns y16, or (y16, y32, psum) when want_y32/want_psum is set."""
    import torch
    M, N = sa.shape[0], sw.shape[0]
    K = sa.shape[1] * 128
    dev = qa6.device
    _need_gpu(qa6, "qa6", torch.uint8, (f6_rows(M), K * 3 // 4), dev)
    _need_gpu(qw6, "qw6", torch.uint8, (f6_rows(N), K * 3 // 4), dev)
    _need_gpu(sa, "s_a", torch.float32, (M, K // 128), dev)
    _need_gpu(sw, "s_w", torch.float32, (N, K // 128), dev)
    if y16 is not None:
        _need_gpu(y16, "y16", torch.float16, (M, N), dev)
    if y32 is not None:
        _need_gpu(y32, "y32", torch.float32, (M, N), dev)
    if y16 is None:
        y16 = torch.empty((M, N), dtype=torch.float16, device=dev)
    if want_y32 and y32 is None:
        y32 = torch.empty((M, N), dtype=torch.float32, device=dev)
    psum = torch.empty((M, N, K // 128), dtype=torch.int32, device=dev) if want_psum else None
    ws_bytes = workspace_size(M, N, K, 128, 128)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    _check("apex4_gemm_w4a4_f6", lib().apex4_gemm_w4a4_f6(
        _ptr(qa6), _ptr(sa), _ptr(qw6), _ptr(sw), M, N, K, _ptr(y16), _ptr(y32), _ptr(psum),
        _ptr(ws), ws_bytes, _stream(torch, dev)))
    if want_y32 or want_psum:
        return y16, y32, psum
    return y16


def select_granularity(M: int, N: int, K: int, min_rel_speed: float = 0.75) -> tuple[int, int]:
    """(group_a, group_w) from apex4_select_granularity (include/apex4.h): the
    finest group mode within min_rel_speed of the fastest one for this shape."""
    ga, gw = ctypes.c_int32(0), ctypes.c_int32(0)
    _check("apex4_select_granularity",
           lib().apex4_select_granularity(M, N, K, min_rel_speed, ctypes.byref(ga), ctypes.byref(gw)))
    return ga.value, gw.value


def _probe(name: str, *args):
    """Run one probe of include/apex4_probe.h on torch's current stream;
    returns the work it reports (operations or bytes)."""
    import torch
    dev = torch.device("cuda", torch.cuda.current_device())
    out = ctypes.c_double(0.0)
    _check(name, getattr(lib(), name)(*args, ctypes.byref(out), _stream(torch, dev)))
    return out.value


def probe_mfma_i8(iters: int, sink) -> float:
    """Independent int8 MFMAs; returns the integer operations issued."""
    _need_gpu(sink, "sink")
    return _probe("apex4_probe_mfma_i8", iters, _ptr(sink))


def probe_mfma_f6(iters: int, sink) -> float:
    """Independent FP6 (E2M3) micro-scaling MFMAs; returns the floating-point operations issued."""
    _need_gpu(sink, "sink")
    return _probe("apex4_probe_mfma_f6", iters, _ptr(sink))


def probe_hbm_read(buf, sink) -> float:
    """Streaming read of the whole of `buf` (a multiple of 4096 bytes); returns the bytes read."""
    _need_gpu(buf, "buf")
    _need_gpu(sink, "sink")
    return _probe("apex4_probe_hbm_read", _ptr(buf), buf.numel() * buf.element_size(), _ptr(sink))


def probe_valu_f32(iters: int, sink) -> float:
    """fp32 FMA chains on the vector ALU; returns the floating-point operations."""
    _need_gpu(sink, "sink")
    return _probe("apex4_probe_valu_f32", iters, _ptr(sink))


def probe_lds_read(iters: int, sink) -> float:
    """16-byte LDS reads, conflict-free; returns the LDS bytes read."""
    _need_gpu(sink, "sink")
    return _probe("apex4_probe_lds_read", iters, _ptr(sink))
