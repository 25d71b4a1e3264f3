"""GPU parity: every entry point of the C ABI against the CPU oracle, bit for bit.

Shapes sweep the row count across both kernel families (split-K small-M
kernel up to 64 rows, LDS-tiled kernels above) and across tile edges, with
ragged N and K tails.  Tolerance is zero: int32 accumulators and block
partials must be equal, fp32 outputs must have equal bit patterns.
"""
import numpy as np
import pytest
import torch

import oracle
from exact_int8_gemm_amd import prism
from exact_int8_gemm_amd import workloads as wl
from gpu_util import DEV, assert_same_floats, assert_same_ints, dev, host

pytestmark = pytest.mark.gpu

M_SWEEP = [1, 2, 3, 7, 8, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257]


# ------------------------------------------------------------------ quantizer

@pytest.mark.parametrize("M,K", [(1, 16), (5, 48), (64, 256), (3, 512), (33, 2560), (8, 9728), (4, 10240),
                                 (4, 10256), (2, 20480), (300, 512), (2, 65536), (2, 65552), (3, 131072),
                                 (1024, 16), (1024, 5120), (1100, 2576), (1030, 20480), (1023, 9728)])
def test_quantize_rows(M, K):
    rng = np.random.default_rng(M * 100003 + K)
    x = rng.standard_normal((M, K), dtype=np.float32)
    x[:, rng.choice(K, max(1, K // 100), replace=False)] *= np.float32(20.0)
    q_ref, s_ref = oracle.quantize_rows(x)
    q, s = prism.quantize_rows(dev(x))
    torch.cuda.synchronize()
    assert_same_floats(host(s), s_ref, "scale")
    assert_same_ints(host(q), q_ref, "codes")


def test_quantize_special_rows():
    K = 64
    rows = []
    rows.append(np.zeros(K))                                   # all zeros
    r = np.zeros(K); r[3] = -0.0; rows.append(r)               # negative zeros
    r = np.ones(K); r[5] = np.nan; rows.append(r)              # NaN
    r = np.ones(K); r[0] = np.inf; rows.append(r)              # +inf
    r = np.ones(K); r[63] = -np.inf; rows.append(r)            # -inf
    rows.append(np.full(K, 1e-44))                             # subnormal amax: scale 0
    rows.append((np.arange(K) - 60) * 3 * 2.0 ** -149)         # subnormal scale, clamp binds
    rows.append(np.linspace(-3e38, 3e38, K))                   # huge values
    r = np.arange(K) - 32 + 0.5; r[0] = 127.0; rows.append(r)  # exact halves with scale 1
    r = np.full(K, 2.5); r[1] = -127.0; rows.append(r)         # ties to even, negative max
    rows.append(np.full(K, 7.0))                               # constant row -> all 127
    x = np.array(rows, dtype=np.float32)
    q_ref, s_ref = oracle.quantize_rows(x)
    q, s = prism.quantize_rows(dev(x))
    torch.cuda.synchronize()
    assert_same_floats(host(s), s_ref, "scale")
    assert_same_ints(host(q), q_ref, "codes")


def _near_tie_rows(rng, rows, K, scale_of_row):
    """Rows whose values sit on and within 4 ulps of the rounding ties (k + 1/2) s of
    their own scale s (the row's absmax, 127 s, is in every row)."""
    x = np.empty((rows, K), np.float32)
    for i in range(rows):
        s = np.float32(scale_of_row(i))
        k = rng.integers(-127, 127, K)
        t = ((k + 0.5) * s.astype(np.float64)).astype(np.float32)
        steps = rng.integers(-4, 5, K)
        for j in range(K):
            v = t[j]
            d = np.float32(np.inf) if steps[j] > 0 else np.float32(-np.inf)
            for _ in range(abs(int(steps[j]))):
                v = np.nextafter(v, d)
            x[i, j] = v
        x[i, 0] = np.float32(127.0) * s
    return x


def test_quantize_near_rounding_ties():
    """Codes next to rounding ties, where multiplying by 1/s and dividing by s can
    round differently: the codes must be those of the correctly rounded quotient."""
    rng = np.random.default_rng(77)
    x = _near_tie_rows(rng, 24, 512, lambda i: rng.uniform(0.5, 1.0) * 2.0 ** int(rng.integers(-20, 20)))
    q_ref, s_ref = oracle.quantize_rows(x)
    q, s = prism.quantize_rows(dev(x))
    torch.cuda.synchronize()
    assert_same_floats(host(s), s_ref, "scale")
    assert_same_ints(host(q), q_ref, "codes")
    for scale in (np.float32(0.0170001), np.float32(3.1e-3)):
        xs = _near_tie_rows(rng, 8, 512, lambda i: scale)
        xs[:, 0] *= np.float32(1.5)   # beyond the range: saturates
        q_ref, s_ref = oracle.quantize_rows_static(xs, float(scale))
        q, s = prism.quantize_rows_static(dev(xs), float(scale))
        torch.cuda.synchronize()
        assert_same_ints(host(q), q_ref, "static codes")


STATIC_SCALES = [0.0625, 0.0170001, 0.0123, 3.0e-3, 2.0 ** -140]


@pytest.mark.parametrize("M,K", [(1, 16), (5, 48), (33, 2560), (8, 9728), (4, 10256), (2, 65552), (3, 131072),
                                 (1100, 2576), (1030, 20480)])
@pytest.mark.parametrize("scale", STATIC_SCALES)
def test_quantize_rows_static(M, K, scale):
    rng = np.random.default_rng(M * 7919 + K)
    x = rng.standard_normal((M, K), dtype=np.float32) * np.float32(0.6)
    x[:, rng.choice(K, max(1, K // 50), replace=False)] *= np.float32(40.0)   # beyond the range: saturate
    # values next to (n + 1/2) * scale: x / scale sits at a rounding tie
    n = rng.integers(-130, 130, size=K)
    t = ((n + 0.5) * np.float32(scale)).astype(np.float32)
    x[0] = np.where(n % 2 == 0, t, np.nextafter(t, np.float32(np.inf) * np.sign(n + 0.5)))
    q_ref, s_ref = oracle.quantize_rows_static(x, scale)
    q, s = prism.quantize_rows_static(dev(x), scale)
    torch.cuda.synchronize()
    assert_same_floats(host(s), s_ref, "scale")
    assert_same_ints(host(q), q_ref, "codes")


@pytest.mark.parametrize("scale", [1.0, 1e-3, 2.0 ** -140, 3.0e38])
def test_quantize_static_special_rows(scale):
    K = 64
    rows = []
    rows.append(np.zeros(K))                                   # all zeros
    r = np.zeros(K); r[3] = -0.0; rows.append(r)               # negative zeros
    r = np.ones(K); r[5] = np.nan; rows.append(r)              # NaN: the row is flagged
    r = np.ones(K); r[0] = np.inf; rows.append(r)              # +inf saturates
    r = np.ones(K); r[63] = -np.inf; rows.append(r)            # -inf saturates
    rows.append(np.full(K, 1e-44))                             # subnormal inputs
    rows.append(np.linspace(-3e38, 3e38, K))                   # huge values: x / s overflows
    r = np.arange(K) - 32 + 0.5; rows.append(r)                # exact halves at scale 1
    r = np.full(K, 2.5); r[1] = -127.5; rows.append(r)         # ties to even, clamp at -127
    x = np.array(rows, dtype=np.float32)
    q_ref, s_ref = oracle.quantize_rows_static(x, scale)
    q, s = prism.quantize_rows_static(dev(x), scale)
    torch.cuda.synchronize()
    assert_same_floats(host(s), s_ref, "scale")
    assert_same_ints(host(q), q_ref, "codes")


def test_static_quantize_then_gemm():
    """Static scale end to end: quantize with the calibrated scale, then the W8A8 GEMM."""
    rng = np.random.default_rng(77)
    M, N, K = 70, 300, 1040
    x = rng.standard_normal((M, K), dtype=np.float32)
    w = wl.int8_weights(rng, N, K)
    s_w = wl.channel_scales(rng, N)
    scale = 0.021
    q_ref, sa_ref = oracle.quantize_rows_static(x, scale)
    y_ref, acc_ref = oracle.gemm_w8a8(q_ref, sa_ref, w, s_w)
    q, sa = prism.quantize_rows_static(dev(x), scale)
    acc = torch.empty((M, N), dtype=torch.int32, device=DEV)
    y = prism.gemm_w8a8(q, sa, dev(w), dev(s_w), acc=acc)
    torch.cuda.synchronize()
    assert_same_ints(host(acc), acc_ref, "acc")
    assert_same_floats(host(y), y_ref, "y")


@pytest.mark.parametrize("bad", [0.0, -2.0, float("inf"), float("nan")])
def test_static_quantize_bad_scale_raises_and_writes_nothing(bad):
    x = dev(np.ones((2, 32), np.float32))
    q = torch.full((2, 32), 5, dtype=torch.int8, device=DEV)
    s = torch.full((2,), 9.0, dtype=torch.float32, device=DEV)
    with pytest.raises(prism.PrismError):
        prism.quantize_rows_static(x, bad, q=q, scale=s)
    torch.cuda.synchronize()
    assert (host(q) == 5).all() and (host(s) == 9.0).all()


# ------------------------------------------------------------------ Q8_0 blocks

@pytest.mark.parametrize("N,K", [(1, 32), (3, 96), (255, 32), (257, 32), (7, 1056), (100, 5120), (17408, 5120)])
def test_repack_q8_0(N, K):
    """Random bytes (any bit pattern is a valid block): every output byte must equal the oracle's."""
    rng = np.random.default_rng(N * 31 + K)
    blocks = rng.integers(0, 256, N * (K // 32) * 34, dtype=np.uint8)
    w_ref, d_ref = oracle.repack_q8_0(blocks, N, K)
    w, d = prism.repack_q8_0(dev(blocks), N, K)
    torch.cuda.synchronize()
    assert_same_ints(host(w), w_ref, "codes")
    assert_same_ints(host(d).view(np.uint16), d_ref, "scales")


def test_repack_q8_0_then_blockscale_gemm():
    """Q8_0 file bytes -> repack -> block-scale GEMM, against the oracle on the same bytes."""
    rng = np.random.default_rng(91)
    M, N, K = 65, 300, 1056
    w = wl.int8_weights(rng, N, K)
    dbits = wl.block_scale_bits(rng, N, K // 32)
    blocks = np.empty((N, K // 32, 34), np.uint8)
    blocks[:, :, 0:2] = dbits.astype("<u2").view(np.uint8).reshape(N, K // 32, 2)
    blocks[:, :, 2:] = w.reshape(N, K // 32, 32).view(np.uint8)
    blocks = blocks.reshape(-1)
    x = rng.standard_normal((M, K), dtype=np.float32)
    q_ref, sa_ref = oracle.quantize_rows(x)
    w_ref, d_ref = oracle.repack_q8_0(blocks, N, K)
    y_ref, _ = oracle.gemm_w8a8_blockscale(q_ref, sa_ref, w_ref, d_ref, False)
    q, sa = prism.quantize_rows(dev(x))
    wg, dg = prism.repack_q8_0(dev(blocks), N, K)
    y = prism.gemm_w8a8_blockscale(q, sa, wg, dg)
    torch.cuda.synchronize()
    assert_same_floats(host(y), y_ref, "y")


# ------------------------------------------------------------------ Q4_K blocks

@pytest.mark.parametrize("N,K", [(1, 256), (3, 512), (63, 256), (65, 768), (100, 5120)])
def test_repack_q4_k(N, K):
    """Random bytes: the code and header planes, byte for byte."""
    rng = np.random.default_rng(N * 17 + K)
    blocks = rng.integers(0, 256, N * (K // 256) * 144, dtype=np.uint8)
    w_ref, h_ref = oracle.repack_q4_k(blocks, N, K)
    w4, hdr = prism.repack_q4_k(dev(blocks), N, K)
    torch.cuda.synchronize()
    assert_same_ints(host(w4), w_ref, "packed codes")
    assert_same_ints(host(hdr), h_ref, "headers")


@pytest.mark.parametrize("M", [1, 2, 4, 7, 16, 17, 65, 129, 257])
@pytest.mark.parametrize("N,K", [(100, 256), (300, 1024), (130, 2304)])
def test_gemm_w4a8_q4k(M, N, K):
    """Q4_K bytes -> GPU repack -> GPU GEMM, against the oracle straight from the bytes."""
    from test_oracle_pins import _pack_q4_k, _q4k_case
    codes, d16, dmin16, sc, mn = _q4k_case(M * 1000 + N + K, N, K)
    blocks = _pack_q4_k(codes, d16, dmin16, sc, mn)
    rng = np.random.default_rng(M + 5)
    x = rng.standard_normal((M, K), dtype=np.float32)
    q_ref, sa_ref = oracle.quantize_rows(x)
    y_ref = oracle.gemm_w4a8_q4k(q_ref, sa_ref, blocks, N)
    w4, hdr = prism.repack_q4_k(dev(blocks), N, K)
    y = prism.gemm_w4a8_q4k(dev(q_ref), dev(sa_ref), w4, hdr)
    torch.cuda.synchronize()
    assert_same_floats(host(y), y_ref, "y")


@pytest.mark.parametrize("M", [3, 40])
def test_gemm_w4a8_q4k_on_oracle_planes_with_any_header_bytes(M):
    """The GEMM on planes written by the oracle's repack (not the GPU's), from random
    block bytes: headers with binary16 NaN, infinite, subnormal and zero d and dmin,
    every 6-bit scale and min; rows of zeros and a NaN row of activations."""
    N, K = 70, 768
    rng = np.random.default_rng(M * 3 + 1)
    blocks = rng.integers(0, 256, N * (K // 256) * 144, dtype=np.uint8)
    x = rng.standard_normal((M, K), dtype=np.float32)
    x[1] = 0.0
    x[2, 5] = np.nan
    q_ref, sa_ref = oracle.quantize_rows(x)
    y_ref = oracle.gemm_w4a8_q4k(q_ref, sa_ref, blocks, N)
    w_ref, h_ref = oracle.repack_q4_k(blocks, N, K)
    y = prism.gemm_w4a8_q4k(dev(q_ref), dev(sa_ref), dev(w_ref), dev(h_ref))
    torch.cuda.synchronize()
    assert np.isnan(y_ref).any() and np.isfinite(y_ref).any()
    assert_same_floats(host(y), y_ref, "y")


# ------------------------------------------------------------------ GEMMs

def _case(seed, M, N, K, kind):
    c = wl.random_case(seed, M, N, K, kind)
    q, s_a = oracle.quantize_rows(c["x"])
    return c, q, s_a


@pytest.mark.parametrize("M", M_SWEEP)
@pytest.mark.parametrize("N,K", [(16, 16), (100, 144), (300, 1040)])
def test_w8a8(M, N, K):
    c, q, s_a = _case(1, M, N, K, "w8a8")
    y_ref, acc_ref = oracle.gemm_w8a8(q, s_a, c["w"], c["s_w"])
    acc = torch.empty((M, N), dtype=torch.int32, device=DEV)
    y = prism.gemm_w8a8(dev(q), dev(s_a), dev(c["w"]), dev(c["s_w"]), acc=acc)
    torch.cuda.synchronize()
    assert_same_ints(host(acc), acc_ref, "acc")
    assert_same_floats(host(y), y_ref, "y")


@pytest.mark.parametrize("M", M_SWEEP)
@pytest.mark.parametrize("N,K", [(16, 32), (100, 160), (300, 1056)])
def test_w4a8(M, N, K):
    c, q, s_a = _case(2, M, N, K, "w4a8")
    y_ref, acc_ref = oracle.gemm_w4a8(q, s_a, c["w4"], c["s_w"])
    acc = torch.empty((M, N), dtype=torch.int32, device=DEV)
    y = prism.gemm_w4a8(dev(q), dev(s_a), dev(c["w4"]), dev(c["s_w"]), acc=acc)
    torch.cuda.synchronize()
    assert_same_ints(host(acc), acc_ref, "acc")
    assert_same_floats(host(y), y_ref, "y")


@pytest.mark.parametrize("M", [1, 7, 16, 17, 64, 65, 129, 257])
@pytest.mark.parametrize("N,K", [(16, 32), (100, 160), (300, 1056)])
def test_w8a8_blockscale(M, N, K):
    c, q, s_a = _case(3, M, N, K, "block")
    y_ref, p_ref = oracle.gemm_w8a8_blockscale(q, s_a, c["w"], c["d"], want_partials=True)
    part = torch.empty((M, N, K // 32), dtype=torch.int32, device=DEV)
    y = prism.gemm_w8a8_blockscale(dev(q), dev(s_a), dev(c["w"]), dev(c["d"]), partials=part)
    y2 = prism.gemm_w8a8_blockscale(dev(q), dev(s_a), dev(c["w"]), dev(c["d"]))   # without partials
    torch.cuda.synchronize()
    assert_same_ints(host(part), p_ref, "partials")
    assert_same_floats(host(y), y_ref, "y")
    assert_same_floats(host(y2), y_ref, "y without partials")


@pytest.mark.parametrize("w4", [False, True])
@pytest.mark.parametrize("N,K", [(1, 32), (257, 1024), (1000, 1056), (3000, 4096), (700, 9728), (300, 16384),
                                 (200, 16416), (100, 32768), (90, 32800), (70000, 32)])
def test_single_row(w4, N, K):
    """M = 1: int8 weights take the row-streaming kernel (one output per row,
    rows spread over all waves) up to 16 KB rows and the MFMA kernel past
    that; 4-bit weights the MFMA kernel.  Row-length classes on both sides of
    the hand-over, against the oracle, with -128 codes."""
    rng = np.random.default_rng(N * 7 + K + w4)
    q = rng.integers(-128, 128, (1, K), dtype=np.int8)
    q[0, :8] = -128
    s_a = rng.uniform(1e-3, 1e-2, 1).astype(np.float32)
    s_w = wl.channel_scales(rng, N)
    if w4:
        w = rng.integers(-8, 8, (N, K), dtype=np.int8)
        w[:, :8] = -8
        wp = wl.pack_int4(w)
        y_ref, acc_ref = oracle.gemm_w4a8(q, s_a, wp, s_w)
        acc = torch.empty((1, N), dtype=torch.int32, device=DEV)
        y = prism.gemm_w4a8(dev(q), dev(s_a), dev(wp), dev(s_w), acc=acc)
    else:
        w = rng.integers(-128, 128, (N, K), dtype=np.int8)
        w[:, :8] = -128
        y_ref, acc_ref = oracle.gemm_w8a8(q, s_a, w, s_w)
        acc = torch.empty((1, N), dtype=torch.int32, device=DEV)
        y = prism.gemm_w8a8(dev(q), dev(s_a), dev(w), dev(s_w), acc=acc)
    torch.cuda.synchronize()
    assert_same_ints(host(acc), acc_ref, "acc")
    assert_same_floats(host(y), y_ref, "y")


def _special_row(kind, K, rng):
    x = rng.standard_normal(K).astype(np.float32)
    if kind == "zero":
        x[:] = 0.0
    elif kind == "nan":
        x[K // 3] = np.nan
    elif kind == "inf":
        x[K - 1] = -np.inf
    elif kind == "tiny":          # amax / 127 underflows to a subnormal scale
        x = (x * np.float32(1e-39)).astype(np.float32)
    elif kind == "huge":
        x = (x * np.float32(1e37)).astype(np.float32)
    elif kind == "ties":          # x / s lands on k + 1/2 for s = 1: amax 127
        x[:] = 0.5
        x[0] = 127.0
        x[1::7] = -2.5
    return x


@pytest.mark.parametrize("N,K", [(1, 16), (700, 1024), (300, 1040), (3000, 5120), (2560, 9728), (257, 16384),
                                 (100, 16400), (70000, 32)])
@pytest.mark.parametrize("kind", ["normal", "zero", "nan", "inf", "tiny", "huge", "ties"])
def test_quantize_gemm_single_row(N, K, kind):
    """One call that quantizes x and multiplies (one kernel for M = 1 up to K = 16384, two
    launches past that): y, acc, the codes and the scale equal the oracle's quantize-then-GEMM
    and the library's two separate calls, bit for bit, also for rows the quantizer marks."""
    rng = np.random.default_rng(N + K + len(kind))
    x = _special_row(kind, K, rng)[None, :]
    w = rng.integers(-128, 128, (N, K), dtype=np.int8)
    s_w = wl.channel_scales(rng, N)
    q_ref, s_ref = oracle.quantize_rows(x)
    y_ref, acc_ref = oracle.gemm_w8a8(q_ref, s_ref, w, s_w)
    xd, wd, swd = dev(x), dev(w), dev(s_w)
    acc = torch.empty((1, N), dtype=torch.int32, device=DEV)
    y, q, s = prism.quantize_gemm_w8a8(xd, wd, swd, acc=acc)
    q2, s2 = prism.quantize_rows(xd)
    y2 = prism.gemm_w8a8(q2, s2, wd, swd)
    torch.cuda.synchronize()
    assert_same_ints(host(q), q_ref, "q")
    assert_same_floats(host(s), s_ref, "scale")
    assert_same_ints(host(acc), acc_ref, "acc")
    assert_same_floats(host(y), y_ref, "y")
    assert_same_floats(host(y), host(y2), "y against the two-call path")


@pytest.mark.parametrize("M,N,K", [(2, 300, 1040), (7, 1000, 5120), (100, 257, 2064), (300, 130, 4096)])
def test_quantize_gemm_several_rows(M, N, K):
    c = wl.random_case(M + N + K, M, N, K, "w8a8")
    c["x"][M // 2] = 0.0
    c["x"][M - 1, 5] = np.nan
    q_ref, s_ref = oracle.quantize_rows(c["x"])
    y_ref, acc_ref = oracle.gemm_w8a8(q_ref, s_ref, c["w"], c["s_w"])
    acc = torch.empty((M, N), dtype=torch.int32, device=DEV)
    y, q, s = prism.quantize_gemm_w8a8(dev(c["x"]), dev(c["w"]), dev(c["s_w"]), acc=acc)
    torch.cuda.synchronize()
    assert_same_ints(host(q), q_ref, "q")
    assert_same_floats(host(s), s_ref, "scale")
    assert_same_ints(host(acc), acc_ref, "acc")
    assert_same_floats(host(y), y_ref, "y")


_FUSED_KINDS = ["normal", "zero", "nan", "inf", "tiny", "huge", "ties"]


def _fused_rows(M, K, seed):
    """M >= 2 rows: a zero row first, a NaN row last, and between them rows cycling
    through the quantizer's other cases (ordinary, inf, tiny and huge scales, rounding ties)."""
    rng = np.random.default_rng(seed)
    kinds = ["zero"] + [_FUSED_KINDS[(m + seed) % len(_FUSED_KINDS)] for m in range(1, M - 1)] + ["nan"]
    return np.stack([_special_row(k, K, rng) for k in kinds])


@pytest.mark.parametrize("M", [2, 3, 4, 5, 7, 8, 9, 16])
@pytest.mark.parametrize("N,K", [(9728, 2560), (2560, 9728), (300, 1040), (3, 16), (5, 2064), (16384, 6144),
                                 (257, 10240), (1000, 14336), (16384, 32), (16400, 1024), (4000, 4096)])
def test_quantize_gemm_few_rows(M, N, K):
    """2..16 rows through the one call: M = 2, 3, 4 as one kernel in which every workgroup
    quantizes the rows itself (the projection shapes, ragged N and K, N < M, the largest N
    and K), more rows, longer rows or N > 16384 as two launches.  Codes, scales, acc and y equal the
    oracle's quantize-then-GEMM and the library's two separate calls, bit for bit, with zero
    and NaN rows among them."""
    rng = np.random.default_rng(M * 7919 + N + K)
    x = _fused_rows(M, K, M + N + K)
    w = rng.integers(-128, 128, (N, K), dtype=np.int8)
    s_w = wl.channel_scales(rng, N)
    q_ref, s_ref = oracle.quantize_rows(x)
    y_ref, acc_ref = oracle.gemm_w8a8(q_ref, s_ref, w, s_w)
    xd, wd, swd = dev(x), dev(w), dev(s_w)
    acc = torch.empty((M, N), dtype=torch.int32, device=DEV)
    y, q, s = prism.quantize_gemm_w8a8(xd, wd, swd, acc=acc)
    q2, s2 = prism.quantize_rows(xd)
    y2 = prism.gemm_w8a8(q2, s2, wd, swd)
    torch.cuda.synchronize()
    assert np.isnan(s_ref).any() and (s_ref == 0).any()
    assert_same_ints(host(q), q_ref, "q")
    assert_same_floats(host(s), s_ref, "scale")
    assert_same_ints(host(acc), acc_ref, "acc")
    assert_same_floats(host(y), y_ref, "y")
    assert_same_floats(host(y), host(y2), "y against the two-call path")


@pytest.mark.parametrize("M,K", [(2, 14336), (2, 14352), (3, 10240), (3, 10256), (4, 6144), (4, 6160)])
def test_quantize_gemm_few_rows_at_the_one_kernel_k_limit(M, K):
    """The longest rows the one-kernel form takes for 2, 3 and 4 rows, and 16 more (two
    launches): bit-exact against the oracle either way."""
    N = 700
    rng = np.random.default_rng(M + K)
    x = _fused_rows(M, K, K)
    w = rng.integers(-128, 128, (N, K), dtype=np.int8)
    s_w = wl.channel_scales(rng, N)
    q_ref, s_ref = oracle.quantize_rows(x)
    y_ref, acc_ref = oracle.gemm_w8a8(q_ref, s_ref, w, s_w)
    acc = torch.empty((M, N), dtype=torch.int32, device=DEV)
    y, q, s = prism.quantize_gemm_w8a8(dev(x), dev(w), dev(s_w), acc=acc)
    torch.cuda.synchronize()
    assert_same_ints(host(q), q_ref, "q")
    assert_same_floats(host(s), s_ref, "scale")
    assert_same_ints(host(acc), acc_ref, "acc")
    assert_same_floats(host(y), y_ref, "y")


def test_quantize_gemm_few_rows_back_to_back_and_two_streams():
    """Calls of different row counts in a row on one stream, then the same calls on a second
    stream while the first one runs them too: all equal the oracle bit for bit."""
    N, K = 2560, 9728
    rng = np.random.default_rng(5)
    w = rng.integers(-128, 128, (N, K), dtype=np.int8)
    s_w = wl.channel_scales(rng, N)
    wd, swd = dev(w), dev(s_w)
    cases = [(M, _fused_rows(M, K, 40 + M)) for M in (4, 2, 9, 16, 3)]
    refs = [oracle.gemm_w8a8(*oracle.quantize_rows(x), w, s_w)[0] for _, x in cases]
    outs = [prism.quantize_gemm_w8a8(dev(x), wd, swd)[0] for _, x in cases]
    side = torch.cuda.Stream(device=DEV)
    xs = [dev(x) for _, x in cases]
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        outs_side = [prism.quantize_gemm_w8a8(x, wd, swd)[0] for x in xs]
    outs_main = [prism.quantize_gemm_w8a8(x, wd, swd)[0] for x in xs]
    torch.cuda.synchronize()
    for i, ref in enumerate(refs):
        assert_same_floats(host(outs[i]), ref, "call %d" % i)
        assert_same_floats(host(outs_side[i]), ref, "side stream, call %d" % i)
        assert_same_floats(host(outs_main[i]), ref, "main stream beside it, call %d" % i)


def test_full_int8_range_and_largest_k():
    """-128 codes and weights (valid inputs, though the quantizer never makes -128)
    and the largest accepted K: the exact sums reach K * 16384 < 2^31."""
    K = prism.K_MAX
    M, N = 4, 3
    q = np.full((M, K), -128, np.int8)
    q[1] = 127
    q[2] = np.tile(np.array([-128, 127], np.int8), K // 2)
    q[3] = 1
    w = np.full((N, K), -128, np.int8)
    w[1] = 127
    w[2, ::2] = 0
    s_a = np.array([1.0, 0.5, 2.0 ** -20, 3.0], np.float32)
    s_w = np.array([1.0, 2.0 ** -30, 0.25], np.float32)
    y_ref, acc_ref = oracle.gemm_w8a8(q, s_a, w, s_w)
    acc = torch.empty((M, N), dtype=torch.int32, device=DEV)
    y = prism.gemm_w8a8(dev(q), dev(s_a), dev(w), dev(s_w), acc=acc)
    torch.cuda.synchronize()
    assert int(acc_ref[0, 0]) == K * 16384
    assert_same_ints(host(acc), acc_ref, "acc")
    assert_same_floats(host(y), y_ref, "y")
    # same rows through the tiled kernels (row count above the small-M limit)
    rep = 40
    qb, sab = np.tile(q, (rep, 1)), np.tile(s_a, rep)
    yb_ref = np.tile(y_ref, (rep, 1))
    yb = prism.gemm_w8a8(dev(qb), dev(sab), dev(w), dev(s_w))
    torch.cuda.synchronize()
    assert_same_floats(host(yb), yb_ref, "y tiled")


def test_w4a8_extremes():
    K = 4096
    M, N = 3, 4
    q = np.full((M, K), -128, np.int8)
    q[1] = 127
    q[2] = -127
    wv = np.full((N, K), -8, np.int8)
    wv[1] = 7
    wv[2, 1::2] = 7
    wv[3] = 0
    w4 = wl.pack_int4(wv)
    s_a = np.ones(M, np.float32)
    s_w = np.ones(N, np.float32)
    y_ref, acc_ref = oracle.gemm_w4a8(q, s_a, w4, s_w)
    for rows in (M, 100):  # small-M kernel and tiled kernel
        qq = np.tile(q, (rows // M + 1, 1))[:rows]
        acc = torch.empty((rows, N), dtype=torch.int32, device=DEV)
        prism.gemm_w4a8(dev(qq), dev(np.ones(rows, np.float32)), dev(w4), dev(s_w), acc=acc)
        torch.cuda.synchronize()
        assert_same_ints(host(acc)[:M], acc_ref, "acc rows=%d" % rows)


@pytest.mark.parametrize("M,N,K", [(1, 1, 256), (1, 15, 768), (1, 17, 4096), (1, 300, 2560), (1, 33, 16384),
                                   (1, 20, 16640), (1, 40, 1056), (2, 1, 256), (2, 71, 16384), (2, 30, 16640),
                                   (3, 33, 2560), (4, 129, 8192), (4, 20, 8448), (4, 9, 1056)])
def test_blockscale_few_rows(M, N, K):
    """1 to 4 rows (the per-wave block kernel for K % 256 == 0 and K <= 16384 at M = 1, M K
    <= 32768 otherwise; longer or ragged rows take the M <= 16 kernel): every output
    against the oracle, with full-range codes and weights (-128 included) and scales from
    the whole finite binary16 range."""
    rng = np.random.default_rng(M * 1000 + N * 7 + K)
    q = rng.integers(-128, 128, (M, K), dtype=np.int8)
    w = rng.integers(-128, 128, (N, K), dtype=np.int8)
    d = rng.integers(0, 0x7c00, (N, K // 32), dtype=np.uint16)   # finite, both signs below
    d |= (rng.integers(0, 2, d.shape) << 15).astype(np.uint16)
    s_a = (np.float32(0.0123) * (1 + np.arange(M))).astype(np.float32)
    y_ref, _ = oracle.gemm_w8a8_blockscale(q, s_a, w, d)
    y = prism.gemm_w8a8_blockscale(dev(q), dev(s_a), dev(w), dev(d))
    torch.cuda.synchronize()
    assert_same_floats(host(y), y_ref, "y")


def test_blockscale_single_row_every_fp16_pattern():
    """K = 256, one row: block b of weight row n has scale pattern 8 n + b, so all 65536
    binary16 patterns (NaN, inf, subnormal, -0) pass through the one-row kernel's fold
    (a row with an infinite scale also holds NaN patterns, so its output is NaN)."""
    N, K = 8192, 256
    rng = np.random.default_rng(3)
    q = rng.integers(-127, 128, (1, K), dtype=np.int8)
    w = rng.integers(-127, 128, (N, K), dtype=np.int8)
    d = np.arange(N * 8, dtype=np.uint32).astype(np.uint16).reshape(N, 8)
    s_a = np.array([1.0], np.float32)
    y_ref, _ = oracle.gemm_w8a8_blockscale(q, s_a, w, d)
    y = prism.gemm_w8a8_blockscale(dev(q), dev(s_a), dev(w), dev(d))
    torch.cuda.synchronize()
    assert np.isnan(y_ref).any() and np.isfinite(y_ref).any()
    assert_same_floats(host(y), y_ref, "y")


def test_blockscale_single_row_scales_not_16_byte_aligned():
    """A scale array that is only 2-byte aligned takes the M <= 16 kernel: same bits."""
    N, K = 50, 512
    rng = np.random.default_rng(8)
    q = rng.integers(-127, 128, (1, K), dtype=np.int8)
    w = rng.integers(-127, 128, (N, K), dtype=np.int8)
    d = (rng.uniform(1e-4, 1e-2, (N, K // 32))).astype(np.float16).view(np.uint16)
    s_a = np.array([0.5], np.float32)
    y_ref, _ = oracle.gemm_w8a8_blockscale(q, s_a, w, d)
    buf = torch.zeros(N * (K // 32) + 1, dtype=torch.int16, device=DEV)
    dd = buf[1:].view(N, K // 32)
    dd.copy_(dev(d.view(np.int16)))
    assert dd.data_ptr() % 16 != 0
    y = prism.gemm_w8a8_blockscale(dev(q), dev(s_a), dev(w), dd)
    torch.cuda.synchronize()
    assert_same_floats(host(y), y_ref, "y")


@pytest.mark.parametrize("M,N,K", [(1, 1, 256), (1, 70, 768), (1, 33, 16384), (1, 20, 16640), (2, 70, 768),
                                   (2, 17, 16384), (3, 41, 2560), (4, 9, 8192), (4, 20, 8448)])
def test_gemm_w4a8_q4k_few_rows_any_header_bytes(M, N, K):
    """1 to 4 rows on planes written by the oracle's repack from random block bytes:
    headers with binary16 NaN, infinite, subnormal and zero d and dmin, every 6-bit scale
    and min; a zero activation row among them."""
    rng = np.random.default_rng(M * 100 + N + K)
    blocks = rng.integers(0, 256, N * (K // 256) * 144, dtype=np.uint8)
    x = rng.standard_normal((M, K), dtype=np.float32)
    if M > 1:
        x[1] = 0.0
    q_ref, sa_ref = oracle.quantize_rows(x)
    y_ref = oracle.gemm_w4a8_q4k(q_ref, sa_ref, blocks, N)
    w_ref, h_ref = oracle.repack_q4_k(blocks, N, K)
    y = prism.gemm_w4a8_q4k(dev(q_ref), dev(sa_ref), dev(w_ref), dev(h_ref))
    torch.cuda.synchronize()
    assert_same_floats(host(y), y_ref, "y")


def test_blockscale_every_fp16_pattern():
    """One output per binary16 bit pattern: y = fmaf(1, d, +0) * 1 = d (NaN stays NaN)."""
    N, K = 65536, 32
    x = np.zeros((1, K), np.float32)
    x[0, 0], x[0, 1] = 1.0, 127.0            # scale 1, codes [1, 127, 0, ...]
    q, s_a = oracle.quantize_rows(x)
    assert s_a[0] == 1.0
    w = np.zeros((N, K), np.int8)
    w[:, 0] = 1                              # P = 1 for every row
    d = np.arange(N, dtype=np.uint32).astype(np.uint16).reshape(N, 1)
    y_ref, _ = oracle.gemm_w8a8_blockscale(q, s_a, w, d)
    y = prism.gemm_w8a8_blockscale(dev(q), dev(s_a), dev(w), dev(d))
    torch.cuda.synchronize()
    assert_same_floats(host(y), y_ref, "y")
    # and the same through a 65-row batch (different tile position of the row)
    qb = np.zeros((65, K), np.int8)
    qb[64] = q[0]
    sab = np.ones(65, np.float32)
    yb = prism.gemm_w8a8_blockscale(dev(qb), dev(sab), dev(w), dev(d))
    torch.cuda.synchronize()
    assert_same_floats(host(yb)[64:65], y_ref, "y row 64")


def test_epilogue_subnormal_outputs():
    """Products that land in the fp32 subnormal range must not be flushed."""
    rng = np.random.default_rng(9)
    M, N, K = 70, 40, 64
    q = rng.integers(-127, 128, (M, K), dtype=np.int8)
    w = rng.integers(-127, 128, (N, K), dtype=np.int8)
    s_a = np.full(M, 2.0 ** -85, np.float32)
    s_w = rng.uniform(1e-3, 1e-2, N).astype(np.float32) * np.float32(2.0 ** -60)
    y_ref, _ = oracle.gemm_w8a8(q, s_a, w, s_w)
    assert (np.abs(y_ref[y_ref != 0]) < 1.2e-38).all()
    for rows in (5, M):
        y = prism.gemm_w8a8(dev(q[:rows]), dev(s_a[:rows]), dev(w), dev(s_w))
        torch.cuda.synchronize()
        assert_same_floats(host(y), y_ref[:rows], "y rows=%d" % rows)


def test_m_zero_is_a_no_op():
    y = torch.full((0, 16), 1.0, device=DEV)
    out = prism.gemm_w8a8(torch.empty((0, 64), dtype=torch.int8, device=DEV),
                          torch.empty((0,), dtype=torch.float32, device=DEV),
                          torch.zeros((16, 64), dtype=torch.int8, device=DEV),
                          torch.ones((16,), dtype=torch.float32, device=DEV), y=y)
    assert out.shape == (0, 16)
    q, s = prism.quantize_rows(torch.empty((0, 32), dtype=torch.float32, device=DEV))
    assert q.shape == (0, 32) and s.shape == (0,)


def test_invalid_shapes_raise_before_launch():
    q = torch.zeros((4, 40), dtype=torch.int8, device=DEV)   # K = 40 is not a multiple of 16
    with pytest.raises(prism.PrismError) as e:
        prism.gemm_w8a8(q, torch.ones(4, device=DEV), torch.zeros((8, 40), dtype=torch.int8, device=DEV),
                        torch.ones(8, device=DEV))
    assert e.value.status == -2


@pytest.mark.parametrize("M,N,K", [(65, 130, 2080), (129, 257, 4128), (100, 2560, 9728)])
def test_w4a8_split_k(M, N, K):
    """The 4-bit tiled path splits K the same way; each partial is shifted back from 16 w exactly."""
    c, q, s_a = _case(8, M, N, K, "w4a8")
    y_ref, acc_ref = oracle.gemm_w4a8(q, s_a, c["w4"], c["s_w"])
    acc = torch.empty((M, N), dtype=torch.int32, device=DEV)
    y = prism.gemm_w4a8(dev(q), dev(s_a), dev(c["w4"]), dev(c["s_w"]), acc=acc)
    torch.cuda.synchronize()
    assert_same_ints(host(acc), acc_ref, "acc")
    assert_same_floats(host(y), y_ref, "y")


@pytest.mark.parametrize("M,N,K", [(65, 130, 2064), (200, 300, 4096), (129, 257, 4112), (100, 2560, 9728)])
def test_w8a8_split_k(M, N, K):
    """Few output tiles and a long K: the tiled path splits K over several
    workgroups whose exact int32 partial tiles are added atomically."""
    c, q, s_a = _case(7, M, N, K, "w8a8")
    y_ref, acc_ref = oracle.gemm_w8a8(q, s_a, c["w"], c["s_w"])
    acc = torch.empty((M, N), dtype=torch.int32, device=DEV)
    y = prism.gemm_w8a8(dev(q), dev(s_a), dev(c["w"]), dev(c["s_w"]), acc=acc)
    y2 = prism.gemm_w8a8(dev(q), dev(s_a), dev(c["w"]), dev(c["s_w"]))
    torch.cuda.synchronize()
    assert_same_ints(host(acc), acc_ref, "acc")
    assert_same_floats(host(y), y_ref, "y")
    assert_same_floats(host(y2), y_ref, "y without acc")
