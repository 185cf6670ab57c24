"""CPU oracle for the W4A4 group-quantized GEMM -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this module.  It wraps the plain C oracle in ``apex4_oracle.c``
(symmetric per-group INT4 quantization, exact integer group sums, fp32
rescale-accumulate in ascending group order, as the APEX4 page's Abstract
describes the pure W4A4 GEMM with group dequantization) through ctypes, with
numpy arrays in and out.  It shares no code with the HIP library and imports
nothing from the package that holds it.

Parity status of each function is stated where it is defined; the pins live in
``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "apex4_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_apex4.so")

# -O2, no fast-math, no contraction into FMA: fp32 arithmetic happens exactly
# in the order the C source spells it.
CFLAGS = ["-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]

OK, ERR_ARG, ERR_NONFINITE, ERR_NOMEM = 0, 1, 2, 3


def build(force: bool = True) -> str:
    """Compile the C oracle into ``oracle/liboracle_apex4.so`` with gcc."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class OracleError(RuntimeError):
    pass


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class Oracle:
    """ctypes view of one build of the C oracle (the default build, or a test variant)."""

    def __init__(self, path: str):
        L = ctypes.CDLL(path)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        L.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_f16_to_f32.restype = ctypes.c_float
        L.oracle_f32_to_f16.argtypes = [ctypes.c_float]
        L.oracle_f32_to_f16.restype = ctypes.c_uint16
        L.oracle_code_at.argtypes = [p, i64]
        L.oracle_code_at.restype = ctypes.c_int
        L.oracle_quantize.argtypes = [p, i64, i64, i64, p, p]
        L.oracle_quantize.restype = ctypes.c_int
        L.oracle_gemm.argtypes = [p, p, i64, p, p, i64, i64, i64, i64, p, p, p]
        L.oracle_gemm.restype = ctypes.c_int
        L.oracle_num_threads.argtypes = []
        L.oracle_num_threads.restype = ctypes.c_int
        self.L = L
        self.path = path

    OracleError = OracleError

    def f16_to_f32(self, h: int) -> float:
        """binary16 bits -> value, from the format definition (pinned against numpy)."""
        return float(self.L.oracle_f16_to_f32(int(h) & 0xFFFF))

    def f32_to_f16(self, x: float) -> int:
        """binary32 -> binary16 bits, round to nearest even (pinned against numpy)."""
        return int(self.L.oracle_f32_to_f16(ctypes.c_float(x)))

    def codes(self, packed: np.ndarray, K: int) -> np.ndarray:
        """Decode packed rows [R, K/2] to int8 codes [R, K] (low nibble = even k)."""
        packed = np.ascontiguousarray(packed, dtype=np.uint8)
        out = np.empty((packed.shape[0], K), dtype=np.int8)
        for r in range(packed.shape[0]):
            base = packed[r].ctypes.data_as(ctypes.c_void_p)
            for k in range(K):
                out[r, k] = self.L.oracle_code_at(base, k)
        return out

    def quantize(self, x: np.ndarray, g: int):
        """Symmetric per-group INT4 quantization of fp16 rows.

        x: float16 [R, K].  Returns (packed uint8 [R, K/2], scales float32 [R, K/g]).
        Raises OracleError on bad sizes or non-finite input.
        """
        x = np.ascontiguousarray(x, dtype=np.float16)
        R, K = x.shape
        q = np.empty((R, K // 2), dtype=np.uint8)
        s = np.empty((R, K // g if g else 0), dtype=np.float32)
        rc = self.L.oracle_quantize(_ptr(x.view(np.uint16)), R, K, g, _ptr(q), _ptr(s))
        if rc != OK:
            raise OracleError(f"oracle_quantize failed with code {rc}")
        return q, s

    def gemm(self, qa, s_a, ga, qw, s_w, gw, K, want_p=False, want_y32=True):
        """Y = sum_j s_a*s_w*P_j over K-groups (see apex4_oracle.c).

        Returns (y16 float16 [M,N], y32 float32 [M,N] or None, p int32 [M,N,G] or None).
        """
        qa = np.ascontiguousarray(qa, dtype=np.uint8)
        qw = np.ascontiguousarray(qw, dtype=np.uint8)
        s_a = np.ascontiguousarray(s_a, dtype=np.float32)
        s_w = np.ascontiguousarray(s_w, dtype=np.float32)
        M, N = qa.shape[0], qw.shape[0]
        G = K // min(ga, gw)
        y16 = np.empty((M, N), dtype=np.uint16)
        y32 = np.empty((M, N), dtype=np.float32) if want_y32 else None
        p = np.empty((M, N, G), dtype=np.int32) if want_p else None
        rc = self.L.oracle_gemm(_ptr(qa), _ptr(s_a), ga, _ptr(qw), _ptr(s_w), gw,
                                M, N, K, _ptr(y16), _ptr(y32), _ptr(p))
        if rc != OK:
            raise OracleError(f"oracle_gemm failed with code {rc}")
        return y16.view(np.float16), y32, p

    def num_threads(self) -> int:
        return int(self.L.oracle_num_threads())


_default = None


def default() -> Oracle:
    """The oracle built from apex4_oracle.c as committed."""
    global _default
    if _default is None:
        if not os.path.exists(_LIB):
            build(force=True)
        _default = Oracle(_LIB)
    return _default


def build_variant(src_text: str, out_path: str) -> Oracle:
    """Compile modified oracle source (used by tests that plant a mistake) and load it."""
    src = out_path + ".c"
    with open(src, "w") as f:
        f.write(src_text)
    subprocess.check_call(["gcc", *CFLAGS, src, "-o", out_path, "-lm"])
    return Oracle(out_path)


def source() -> str:
    with open(_SRC) as f:
        return f.read()


# module-level conveniences bound to the default build
def lib():
    return default().L


def f16_to_f32(h):
    return default().f16_to_f32(h)


def f32_to_f16(x):
    return default().f32_to_f16(x)


def codes(packed, K):
    return default().codes(packed, K)


def quantize(x, g):
    return default().quantize(x, g)


def gemm(*a, **kw):
    return default().gemm(*a, **kw)


def num_threads():
    return default().num_threads()
