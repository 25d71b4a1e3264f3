"""Python binding of libprism (the C ABI in ``include/prism.h``).

Argument marshalling only: tensors are checked for dtype, device, shape,
contiguity and alignment, their device pointers and the current HIP stream
are passed to the C entry points, and a non-zero status raises
:class:`PrismError`.  Every step of the computation runs in the HIP kernels
of ``libprism.so``; there is no fallback of any kind, and a missing library
raises instead of computing elsewhere.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libprism.so")

PRISM_OK = 0
ABI_VERSION = 13
K_MAX = 131040

# Dispatch-table entries of the W8A8 / W4A8 calls (PRISM_VARIANT_* in include/prism.h).
VARIANTS = {"auto": 0, "small_1x4": 1, "small_1x8": 2, "small_1x16": 3, "small_2x4": 4, "small_2x8": 5,
            "small_2x16": 6, "tile_256x256": 7, "tile_256x128": 8, "tile_128x128": 9, "tile_128x128_split2": 10,
            "tile_128x128_split3": 11, "tile_128x128_split4": 12, "small_3x4": 13, "small_3x8": 14,
            "small_4x4": 15, "small_4x8": 16, "tile_256x192": 17, "tile_256x320": 18, "tile_64x128": 19,
            "tile_64x128_split2": 20, "tile_64x128_split3": 21, "tile_64x128_split4": 22, "tile_128x96": 23,
            "tile_128x96_split2": 24, "small_balanced": 25,
            "tile_192x128": 26}


class PrismError(RuntimeError):
    def __init__(self, status: int, text: str):
        super().__init__("prism status %d: %s" % (status, text))
        self.status = status


_lib = None


def _declare(lib):
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.prism_abi_version.restype = i32
    lib.prism_abi_version.argtypes = []
    lib.prism_build_id.restype = ctypes.c_char_p
    lib.prism_build_id.argtypes = []
    lib.prism_status_string.restype = ctypes.c_char_p
    lib.prism_status_string.argtypes = [i32]
    lib.prism_quantize_rows.restype = i32
    lib.prism_quantize_rows.argtypes = [p, p, p, i64, i64, p]
    lib.prism_quantize_rows_static.restype = i32
    lib.prism_quantize_rows_static.argtypes = [p, p, p, ctypes.c_float, i64, i64, p]
    lib.prism_repack_q8_0.restype = i32
    lib.prism_repack_q8_0.argtypes = [p, p, p, i64, i64, p]
    lib.prism_repack_q4_k.restype = i32
    lib.prism_repack_q4_k.argtypes = [p, p, p, i64, i64, p]
    lib.prism_gemm_w4a8_q4k.restype = i32
    lib.prism_gemm_w4a8_q4k.argtypes = [p, p, p, p, p, i64, i64, i64, p]
    lib.prism_quantize_gemm_w8a8.restype = i32
    lib.prism_quantize_gemm_w8a8.argtypes = [p, p, p, p, p, p, p, i64, i64, i64, p]
    for name in ("prism_gemm_w8a8_variant", "prism_gemm_w4a8_variant"):
        fn = getattr(lib, name)
        fn.restype = i32
        fn.argtypes = [p, p, p, p, p, p, i64, i64, i64, i32, p]
    for name in ("prism_gemm_w8a8", "prism_gemm_w8a8_blockscale", "prism_gemm_w4a8"):
        fn = getattr(lib, name)
        fn.restype = i32
        fn.argtypes = [p, p, p, p, p, p, i64, i64, i64, p]
    lib.prism_peak_mfma.restype = i32
    lib.prism_peak_mfma.argtypes = [i64, i32, i32, p, p]
    lib.prism_peak_read.restype = i32
    lib.prism_peak_read.argtypes = [p, i64, p, p]
    lib.prism_peak_fold.restype = i32
    lib.prism_peak_fold.argtypes = [i32, i64, p, p]
    return lib


def lib():
    """The loaded ``libprism.so`` (built with hipcc first if it does not exist yet).

    Raises if the library was built from other sources than the ones next to
    this binding (its build id is the hash of the HIP sources, the header and
    the compile flags), so that a stale binary is never the one under test."""
    global _lib
    if _lib is None:
        from . import build
        if not os.path.exists(LIB_PATH):
            build.build_library()
        loaded = _declare(ctypes.CDLL(LIB_PATH))
        v = loaded.prism_abi_version()
        if v != ABI_VERSION:
            raise RuntimeError("libprism ABI version %d, binding expects %d: rebuild" % (v, ABI_VERSION))
        got, want = loaded.prism_build_id().decode(), build.source_hash()
        if got != want:
            raise RuntimeError("%s was built from other sources (build id %s, sources hash to %s): rebuild it "
                               "with exact_int8_gemm_amd.build.build_library()" % (LIB_PATH, got, want))
        _lib = loaded
    return _lib


def status_string(status: int) -> str:
    return lib().prism_status_string(int(status)).decode()


def _check(status: int):
    if status != PRISM_OK:
        raise PrismError(status, status_string(status))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtype, shape, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if t.device != device:
        raise ValueError("%s must be on %s, got %s" % (name, device, t.device))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _gpu(t, name):
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError("%s must be a tensor on a HIP device" % name)
    return t.device


def quantize_rows(x, q=None, scale=None):
    """x float32 [M, K] on the GPU -> (q int8 [M, K], scale float32 [M])."""
    dev = _gpu(x, "x")
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    M, K = x.shape
    _need(x, "x", torch.float32, (M, K), dev)
    q = torch.empty((M, K), dtype=torch.int8, device=dev) if q is None else _need(q, "q", torch.int8, (M, K), dev)
    scale = torch.empty((M,), dtype=torch.float32, device=dev) if scale is None else \
        _need(scale, "scale", torch.float32, (M,), dev)
    with torch.cuda.device(dev):
        _check(lib().prism_quantize_rows(_ptr(x), _ptr(q), _ptr(scale), M, K, _stream(dev)))
    return q, scale


def quantize_rows_static(x, s, q=None, scale=None):
    """x float32 [M, K] on the GPU and one calibrated scale s > 0 -> (q int8 [M, K], scale float32 [M])."""
    dev = _gpu(x, "x")
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    M, K = x.shape
    _need(x, "x", torch.float32, (M, K), dev)
    q = torch.empty((M, K), dtype=torch.int8, device=dev) if q is None else _need(q, "q", torch.int8, (M, K), dev)
    scale = torch.empty((M,), dtype=torch.float32, device=dev) if scale is None else \
        _need(scale, "scale", torch.float32, (M,), dev)
    with torch.cuda.device(dev):
        _check(lib().prism_quantize_rows_static(_ptr(x), _ptr(q), _ptr(scale), ctypes.c_float(float(s)), M, K,
                                                _stream(dev)))
    return q, scale


def repack_q8_0(blocks, N, K, w=None, d=None):
    """Q8_0 blocks (uint8 tensor of N * K/32 * 34 bytes on the GPU) -> (w int8 [N, K], d int16 [N, K/32]).

    ``d`` holds the binary16 bit patterns of the block scales (the dtype the block-scale GEMM takes)."""
    dev = _gpu(blocks, "blocks")
    N, K = int(N), int(K)
    if K <= 0 or K % 32:
        raise ValueError("K must be a positive multiple of 32")
    _need(blocks, "blocks", torch.uint8, (N * (K // 32) * 34,), dev)
    w = torch.empty((N, K), dtype=torch.int8, device=dev) if w is None else _need(w, "w", torch.int8, (N, K), dev)
    d = torch.empty((N, K // 32), dtype=torch.int16, device=dev) if d is None else \
        _need(d, "d", torch.int16, (N, K // 32), dev)
    with torch.cuda.device(dev):
        _check(lib().prism_repack_q8_0(_ptr(blocks), _ptr(w), _ptr(d), N, K, _stream(dev)))
    return w, d


def repack_q4_k(blocks, N, K, w4=None, hdr=None):
    """Q4_K super-blocks (uint8 tensor of N * K/256 * 144 bytes on the GPU) ->
    (w4 uint8 [N, K/2] packed codes in the file's order, hdr uint8 [N, K/256, 16] super-block headers)."""
    dev = _gpu(blocks, "blocks")
    N, K = int(N), int(K)
    if K <= 0 or K % 256:
        raise ValueError("K must be a positive multiple of 256")
    _need(blocks, "blocks", torch.uint8, (N * (K // 256) * 144,), dev)
    w4 = torch.empty((N, K // 2), dtype=torch.uint8, device=dev) if w4 is None else \
        _need(w4, "w4", torch.uint8, (N, K // 2), dev)
    hdr = torch.empty((N, K // 256, 16), dtype=torch.uint8, device=dev) if hdr is None else \
        _need(hdr, "hdr", torch.uint8, (N, K // 256, 16), dev)
    with torch.cuda.device(dev):
        _check(lib().prism_repack_q4_k(_ptr(blocks), _ptr(w4), _ptr(hdr), N, K, _stream(dev)))
    return w4, hdr


def gemm_w4a8_q4k(q, s_a, w4, hdr, y=None):
    """Q4_K-native W4A8: q int8 [M,K], s_a f32 [M], w4 uint8 [N,K/2] packed codes, hdr uint8 [N,K/256,16]
    -> y f32 [M,N]."""
    dev, M, N, K = _gemm_args(q, s_a, w4, lambda k: k // 2, torch.uint8, "hdr", hdr, torch.uint8,
                              lambda n, k: (n, k // 256, 16))
    y = torch.empty((M, N), dtype=torch.float32, device=dev) if y is None else _need(y, "y", torch.float32, (M, N), dev)
    with torch.cuda.device(dev):
        _check(lib().prism_gemm_w4a8_q4k(_ptr(q), _ptr(s_a), _ptr(w4), _ptr(hdr), _ptr(y), M, N, K, _stream(dev)))
    return y


def _gemm_args(q, s_a, w, w_cols, wdtype, s_w_name, s_w, s_w_dtype, s_w_shape_fn):
    dev = _gpu(q, "q")
    if q.dim() != 2 or w.dim() != 2:
        raise ValueError("q and w must be 2-D")
    M, K = q.shape
    N = w.shape[0]
    _need(q, "q", torch.int8, (M, K), dev)
    _need(s_a, "s_a", torch.float32, (M,), dev)
    _need(w, "w", wdtype, (N, w_cols(K)), dev)
    _need(s_w, s_w_name, s_w_dtype, s_w_shape_fn(N, K), dev)
    return dev, M, N, K


def gemm_w8a8(q, s_a, w, s_w, y=None, acc=None):
    """Per-channel W8A8: q int8 [M,K], s_a f32 [M], w int8 [N,K], s_w f32 [N] -> y f32 [M,N].

    If ``acc`` (int32 [M,N]) is given, the exact int32 sums are written there too."""
    dev, M, N, K = _gemm_args(q, s_a, w, lambda k: k, torch.int8, "s_w", s_w, torch.float32, lambda n, k: (n,))
    y = torch.empty((M, N), dtype=torch.float32, device=dev) if y is None else _need(y, "y", torch.float32, (M, N), dev)
    if acc is not None:
        _need(acc, "acc", torch.int32, (M, N), dev)
    with torch.cuda.device(dev):
        _check(lib().prism_gemm_w8a8(_ptr(q), _ptr(s_a), _ptr(w), _ptr(s_w), _ptr(y), _ptr(acc), M, N, K,
                                     _stream(dev)))
    return y


def gemm_w8a8_variant(q, s_a, w, s_w, variant, y=None, acc=None):
    """gemm_w8a8 through one named dispatch-table entry (``VARIANTS``); for verifying that every
    entry gives the same bits."""
    dev, M, N, K = _gemm_args(q, s_a, w, lambda k: k, torch.int8, "s_w", s_w, torch.float32, lambda n, k: (n,))
    y = torch.empty((M, N), dtype=torch.float32, device=dev) if y is None else _need(y, "y", torch.float32, (M, N), dev)
    if acc is not None:
        _need(acc, "acc", torch.int32, (M, N), dev)
    with torch.cuda.device(dev):
        _check(lib().prism_gemm_w8a8_variant(_ptr(q), _ptr(s_a), _ptr(w), _ptr(s_w), _ptr(y), _ptr(acc), M, N, K,
                                             VARIANTS[variant], _stream(dev)))
    return y


def gemm_w4a8_variant(q, s_a, w4, s_w, variant, y=None, acc=None):
    """gemm_w4a8 through one named dispatch-table entry (``VARIANTS``)."""
    dev, M, N, K = _gemm_args(q, s_a, w4, lambda k: k // 2, torch.uint8, "s_w", s_w, torch.float32,
                              lambda n, k: (n,))
    y = torch.empty((M, N), dtype=torch.float32, device=dev) if y is None else _need(y, "y", torch.float32, (M, N), dev)
    if acc is not None:
        _need(acc, "acc", torch.int32, (M, N), dev)
    with torch.cuda.device(dev):
        _check(lib().prism_gemm_w4a8_variant(_ptr(q), _ptr(s_a), _ptr(w4), _ptr(s_w), _ptr(y), _ptr(acc), M, N, K,
                                             VARIANTS[variant], _stream(dev)))
    return y


def quantize_gemm_w8a8(x, w, s_w, y=None, q=None, scale=None, acc=None):
    """Quantize x f32 [M,K] per row and multiply by int8 w [N,K] with s_w f32 [N] in one call:
    the bits of ``quantize_rows`` then ``gemm_w8a8``.  Returns (y, q, scale); q and scale are
    the quantizer's outputs.  M = 1 (decode) and M = 2..4 with N <= 16384 and K up to
    14336 / 10240 / 6144 run as one kernel."""
    dev = _gpu(x, "x")
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    M, K = x.shape
    _need(x, "x", torch.float32, (M, K), dev)
    q = torch.empty((M, K), dtype=torch.int8, device=dev) if q is None else _need(q, "q", torch.int8, (M, K), dev)
    scale = (torch.empty((M,), dtype=torch.float32, device=dev) if scale is None
             else _need(scale, "scale", torch.float32, (M,), dev))
    dev, M, N, K = _gemm_args(q, scale, w, lambda k: k, torch.int8, "s_w", s_w, torch.float32, lambda n, k: (n,))
    y = torch.empty((M, N), dtype=torch.float32, device=dev) if y is None else _need(y, "y", torch.float32, (M, N), dev)
    if acc is not None:
        _need(acc, "acc", torch.int32, (M, N), dev)
    with torch.cuda.device(dev):
        _check(lib().prism_quantize_gemm_w8a8(_ptr(x), _ptr(q), _ptr(scale), _ptr(w), _ptr(s_w), _ptr(y), _ptr(acc),
                                              M, N, K, _stream(dev)))
    return y, q, scale


def gemm_w4a8(q, s_a, w4, s_w, y=None, acc=None):
    """W4A8: q int8 [M,K], s_a f32 [M], w4 uint8 [N,K/2] (low nibble = even k), s_w f32 [N] -> y f32 [M,N]."""
    dev, M, N, K = _gemm_args(q, s_a, w4, lambda k: k // 2, torch.uint8, "s_w", s_w, torch.float32,
                              lambda n, k: (n,))
    y = torch.empty((M, N), dtype=torch.float32, device=dev) if y is None else _need(y, "y", torch.float32, (M, N), dev)
    if acc is not None:
        _need(acc, "acc", torch.int32, (M, N), dev)
    with torch.cuda.device(dev):
        _check(lib().prism_gemm_w4a8(_ptr(q), _ptr(s_a), _ptr(w4), _ptr(s_w), _ptr(y), _ptr(acc), M, N, K,
                                     _stream(dev)))
    return y


def gemm_w8a8_blockscale(q, s_a, w, d, y=None, partials=None):
    """Block-scale W8A8: q int8 [M,K], s_a f32 [M], w int8 [N,K], d [N,K/32] fp16 scales
    (torch.float16, or their bit patterns as int16/uint16) -> y f32 [M,N].

    If ``partials`` (int32 [M,N,K/32]) is given, every exact 32-k block sum is written there."""
    if not isinstance(d, torch.Tensor) or d.dtype not in (torch.float16, torch.int16, torch.uint16):
        raise TypeError("d must be a float16 (or 16-bit integer bit-pattern) tensor")
    dev, M, N, K = _gemm_args(q, s_a, w, lambda k: k, torch.int8, "d", d, d.dtype, lambda n, k: (n, k // 32))
    y = torch.empty((M, N), dtype=torch.float32, device=dev) if y is None else _need(y, "y", torch.float32, (M, N), dev)
    if partials is not None:
        _need(partials, "partials", torch.int32, (M, N, K // 32), dev)
    with torch.cuda.device(dev):
        _check(lib().prism_gemm_w8a8_blockscale(_ptr(q), _ptr(s_a), _ptr(w), _ptr(d), _ptr(y), _ptr(partials),
                                                M, N, K, _stream(dev)))
    return y


# ------------------------------------------------------------ measurement kernels

PEAK_READ_PARTS = 4096


def peak_mfma(iters, waves_per_simd, seed=0, out=None, device=None):
    """Run the MFMA throughput kernel (int8 32x32x32 on registers, no memory traffic):
    2 x CUs workgroups of 2 x waves_per_simd waves, iters x 16 MFMAs per wave.  Returns
    the per-thread checksums (uint32 as int32 [2 * CUs * 128 * waves_per_simd])."""
    dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
    n = 2 * torch.cuda.get_device_properties(dev).multi_processor_count * 128 * waves_per_simd
    out = torch.empty((n,), dtype=torch.int32, device=dev) if out is None else _need(out, "out", torch.int32, (n,), dev)
    with torch.cuda.device(dev):
        _check(lib().prism_peak_mfma(iters, waves_per_simd, seed, _ptr(out), _stream(dev)))
    return out


FOLD_MODES = ("i8_mfma_cvt_fold", "f16_mfma_fold", "i8_mfma_only", "f16_mfma_only", "fold_only")
FOLD_TILES = 5


def peak_fold(mode, iters, out=None, device=None):
    """Run the block-fold probe (one workgroup of 8 waves per CU, 5 tiles of 32 x 32 per
    wave, one 32-k block per tile per iteration) in ``mode`` (index into FOLD_MODES).
    Returns the per-thread sums (float32 [CUs * 512])."""
    dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
    n = torch.cuda.get_device_properties(dev).multi_processor_count * 512
    out = (torch.empty((n,), dtype=torch.float32, device=dev) if out is None
           else _need(out, "out", torch.float32, (n,), dev))
    with torch.cuda.device(dev):
        _check(lib().prism_peak_fold(mode, iters, _ptr(out), _stream(dev)))
    return out


def peak_read(buf, parts=None):
    """Read the bytes of the contiguous CUDA tensor ``buf`` once (16-byte loads); returns
    parts (int32 [PEAK_READ_PARTS]) whose XOR is the XOR of the buffer's 32-bit words."""
    dev = _gpu(buf, "buf")
    if not buf.is_contiguous():
        raise ValueError("buf must be contiguous")
    nbytes = buf.numel() * buf.element_size()
    parts = (torch.empty((PEAK_READ_PARTS,), dtype=torch.int32, device=dev) if parts is None
             else _need(parts, "parts", torch.int32, (PEAK_READ_PARTS,), dev))
    with torch.cuda.device(dev):
        _check(lib().prism_peak_read(_ptr(buf), nbytes, _ptr(parts), _stream(dev)))
    return parts
