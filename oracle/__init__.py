"""CPU oracle for the exact int8 linear layer (ctypes binding of ``oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The GPU library neither imports nor
links anything here, and nothing here imports the GPU library.

The arithmetic lives in ``oracle.c`` (plain int64 triple loops and a fixed
fp32 epilogue; see its header for the readings of the StartLux-Prism README
it follows).  This module only builds the shared object with gcc, marshals
numpy arrays and raises on a non-zero status.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# -ffp-contract=off: every fp32 multiply and add is rounded on its own, as the
# epilogue's definition requires; fmaf() is the only fused operation.
CFLAGS = ["-O2", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-std=c11"]

STATUS = {0: "ok", -1: "invalid argument", -5: "exact sum outside the int32 range"}


class OracleError(RuntimeError):
    pass


def build(force: bool = False) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` next to it (gcc)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def bind(lib):
    """Declare the C signatures on a loaded ``ctypes.CDLL`` of ``oracle.c``."""
    p, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_f16_to_f32.restype = ctypes.c_float
    lib.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_f32_array.restype = None
    lib.oracle_f16_to_f32_array.argtypes = [p, p, i64]
    lib.oracle_quantize_rows.restype = ctypes.c_int
    lib.oracle_quantize_rows.argtypes = [p, p, p, i64, i64]
    lib.oracle_quantize_rows_static.restype = ctypes.c_int
    lib.oracle_quantize_rows_static.argtypes = [p, p, p, ctypes.c_float, i64, i64]
    lib.oracle_repack_q8_0.restype = ctypes.c_int
    lib.oracle_repack_q8_0.argtypes = [p, p, p, i64, i64]
    lib.oracle_repack_q4_k.restype = ctypes.c_int
    lib.oracle_repack_q4_k.argtypes = [p, p, p, i64, i64]
    lib.oracle_gemm_w4a8_q4k.restype = ctypes.c_int
    lib.oracle_gemm_w4a8_q4k.argtypes = [p, p, p, p, i64, i64, i64]
    for name in ("oracle_gemm_w8a8", "oracle_gemm_w4a8", "oracle_gemm_w8a8_blockscale"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [p, p, p, p, p, p, i64, i64, i64]
    return lib


def _load():
    global _lib
    if _lib is None:
        _lib = bind(ctypes.CDLL(build()))
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(status):
    if status != 0:
        raise OracleError(STATUS.get(status, "status %d" % status))


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError("expected %s, got %s" % (np.dtype(dtype), a.dtype))
    return a


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def f16_to_f32(bits) -> np.ndarray:
    """binary16 bit patterns (uint16) -> float32 values."""
    bits = _c(np.asarray(bits), np.uint16)
    out = np.empty(bits.shape, np.float32)
    _load().oracle_f16_to_f32_array(_ptr(bits), _ptr(out), bits.size)
    return out


def quantize_rows(x):
    """x float32 [M, K] -> (q int8 [M, K], s float32 [M])."""
    x = _c(x, np.float32)
    M, K = x.shape
    q = np.empty((M, K), np.int8)
    s = np.empty((M,), np.float32)
    _check(_load().oracle_quantize_rows(_ptr(x), _ptr(q), _ptr(s), M, K))
    return q, s


def quantize_rows_static(x, scale):
    """x float32 [M, K], one static fp32 scale -> (q int8 [M, K], s float32 [M])."""
    x = _c(x, np.float32)
    M, K = x.shape
    q = np.empty((M, K), np.int8)
    s = np.empty((M,), np.float32)
    _check(_load().oracle_quantize_rows_static(_ptr(x), _ptr(q), _ptr(s), ctypes.c_float(scale), M, K))
    return q, s


def repack_q8_0(blocks, N, K):
    """Q8_0 blocks (uint8, N * K/32 * 34 bytes) -> (w int8 [N, K], d uint16 [N, K/32] binary16 bits)."""
    blocks = _c(blocks, np.uint8).reshape(-1)
    assert blocks.size == N * (K // 32) * 34
    w = np.empty((N, K), np.int8)
    d = np.empty((N, K // 32), np.uint16)
    _check(_load().oracle_repack_q8_0(_ptr(blocks), _ptr(w), _ptr(d), N, K))
    return w, d


def repack_q4_k(blocks, N, K):
    """Q4_K blocks (uint8, N * K/256 * 144 bytes) -> (w4 uint8 [N, K/2] packed codes,
    hdr uint8 [N, K/256, 16] super-block headers)."""
    blocks = _c(blocks, np.uint8).reshape(-1)
    assert blocks.size == N * (K // 256) * 144
    w4 = np.empty((N, K // 2), np.uint8)
    hdr = np.empty((N, K // 256, 16), np.uint8)
    _check(_load().oracle_repack_q4_k(_ptr(blocks), _ptr(w4), _ptr(hdr), N, K))
    return w4, hdr


def gemm_w4a8_q4k(q, s_a, blocks, N):
    """q int8 [M, K], s_a f32 [M], Q4_K blocks of an [N, K] weight matrix -> y f32 [M, N]."""
    q, s_a = _c(q, np.int8), _c(s_a, np.float32)
    blocks = _c(blocks, np.uint8).reshape(-1)
    M, K = q.shape
    assert blocks.size == N * (K // 256) * 144 and s_a.shape == (M,)
    y = np.empty((M, N), np.float32)
    _check(_load().oracle_gemm_w4a8_q4k(_ptr(q), _ptr(s_a), _ptr(blocks), _ptr(y), M, N, K))
    return y


def gemm_w8a8(q, s_a, w, s_w):
    """q int8 [M,K], s_a f32 [M], w int8 [N,K], s_w f32 [N] -> (y f32 [M,N], acc i32 [M,N])."""
    q, s_a, w, s_w = _c(q, np.int8), _c(s_a, np.float32), _c(w, np.int8), _c(s_w, np.float32)
    M, K = q.shape
    N = w.shape[0]
    assert w.shape == (N, K) and s_a.shape == (M,) and s_w.shape == (N,)
    y = np.empty((M, N), np.float32)
    acc = np.empty((M, N), np.int32)
    _check(_load().oracle_gemm_w8a8(_ptr(q), _ptr(s_a), _ptr(w), _ptr(s_w), _ptr(y), _ptr(acc), M, N, K))
    return y, acc


def gemm_w4a8(q, s_a, w4, s_w):
    """q int8 [M,K], s_a f32 [M], w4 uint8 [N,K/2], s_w f32 [N] -> (y, acc)."""
    q, s_a, w4, s_w = _c(q, np.int8), _c(s_a, np.float32), _c(w4, np.uint8), _c(s_w, np.float32)
    M, K = q.shape
    N = w4.shape[0]
    assert w4.shape == (N, K // 2) and s_a.shape == (M,) and s_w.shape == (N,)
    y = np.empty((M, N), np.float32)
    acc = np.empty((M, N), np.int32)
    _check(_load().oracle_gemm_w4a8(_ptr(q), _ptr(s_a), _ptr(w4), _ptr(s_w), _ptr(y), _ptr(acc), M, N, K))
    return y, acc


def gemm_w8a8_blockscale(q, s_a, w, d_bits, want_partials=False):
    """q int8 [M,K], s_a f32 [M], w int8 [N,K], d_bits uint16 [N,K/32] (binary16 patterns)
    -> (y f32 [M,N], partials i32 [M,N,K/32] or None)."""
    q, s_a, w, d_bits = _c(q, np.int8), _c(s_a, np.float32), _c(w, np.int8), _c(d_bits, np.uint16)
    M, K = q.shape
    N = w.shape[0]
    assert w.shape == (N, K) and d_bits.shape == (N, K // 32) and s_a.shape == (M,)
    y = np.empty((M, N), np.float32)
    part = np.empty((M, N, K // 32), np.int32) if want_partials else None
    _check(_load().oracle_gemm_w8a8_blockscale(_ptr(q), _ptr(s_a), _ptr(w), _ptr(d_bits), _ptr(y),
                                               _ptr(part), M, N, K))
    return y, part
