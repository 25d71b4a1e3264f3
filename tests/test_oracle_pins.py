"""Pins of the CPU oracle against things other than itself (runs without a GPU).

Every check here comes from outside the oracle's code: Python integers (brute
force), exact rationals (``fractions.Fraction``), numpy's int64 matmul and
binary16 conversion, hand-worked cases in ``golden/hand_cases.json``, and
invariants that the definition of an exact integer sum implies.  A dropped
term, a wrong sign or index, a transposed operand, a wrong rounding mode or a
fused epilogue in the oracle makes at least one of these fail (see
``test_oracle_mutants.py``, which plants such mistakes on purpose).

Definitions followed (StartLux-Prism README): "Why StartLux-Prism" (int8 GEMMs
summed exactly in int32; Q8_0 as W8A8, Q4_K_M as W4A8) and "How it works"
(int8 tensor cores with exact int32 sums); readings as in the oracle header.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from exact import bits, frac, rint_half_even, round_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")


def _rng(seed):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------- accumulators

def _brute_acc(q, w):
    M, K = q.shape
    N = w.shape[0]
    out = [[0] * N for _ in range(M)]
    for m in range(M):
        qa = [int(v) for v in q[m]]
        for n in range(N):
            wa = [int(v) for v in w[n]]
            out[m][n] = sum(a * b for a, b in zip(qa, wa))
    return np.array(out, dtype=np.int64)


def _decode_w4_brute(w4, K):
    """Independent decode: enumerate all 256 (low, high) value pairs in [-8,7]^2
    by the packing rule, then look each byte up."""
    table = {}
    for lo in range(-8, 8):
        for hi in range(-8, 8):
            table[(lo & 15) | ((hi & 15) << 4)] = (lo, hi)
    N = w4.shape[0]
    out = np.zeros((N, K), np.int64)
    for n in range(N):
        for j in range(K // 2):
            lo, hi = table[int(w4[n, j])]
            out[n, 2 * j], out[n, 2 * j + 1] = lo, hi
    return out


@pytest.mark.parametrize("M,N,K,seed", [(1, 1, 1, 0), (3, 5, 7, 1), (8, 8, 128, 2), (5, 3, 96, 3)])
def test_w8a8_acc_brute_force(M, N, K, seed):
    r = _rng(seed)
    q = r.integers(-128, 128, (M, K), dtype=np.int8)
    w = r.integers(-128, 128, (N, K), dtype=np.int8)
    _, acc = oracle.gemm_w8a8(q, np.ones(M, np.float32), w, np.ones(N, np.float32))
    assert np.array_equal(acc.astype(np.int64), _brute_acc(q, w))


@pytest.mark.parametrize("M,N,K,seed", [(1, 1, 2, 0), (4, 6, 64, 1), (8, 8, 128, 2)])
def test_w4a8_acc_brute_force(M, N, K, seed):
    r = _rng(seed)
    q = r.integers(-127, 128, (M, K), dtype=np.int8)
    w4 = r.integers(0, 256, (N, K // 2), dtype=np.uint8)
    _, acc = oracle.gemm_w4a8(q, np.ones(M, np.float32), w4, np.ones(N, np.float32))
    assert np.array_equal(acc.astype(np.int64), _brute_acc(q, _decode_w4_brute(w4, K)))


def test_w8a8_acc_vs_numpy_int64_matmul():
    r = _rng(10)
    M, N, K = 37, 61, 1040
    q = r.integers(-127, 128, (M, K), dtype=np.int8)
    w = r.integers(-127, 128, (N, K), dtype=np.int8)
    _, acc = oracle.gemm_w8a8(q, np.ones(M, np.float32), w, np.ones(N, np.float32))
    ref = q.astype(np.int64) @ w.astype(np.int64).T
    assert np.array_equal(acc.astype(np.int64), ref)


def test_int8_product_table_exhaustive():
    """All 256 x 256 int8 products, one k each."""
    vals = np.arange(-128, 128, dtype=np.int64)
    q = vals.astype(np.int8).reshape(256, 1)
    w = vals.astype(np.int8).reshape(256, 1)
    _, acc = oracle.gemm_w8a8(q, np.ones(256, np.float32), w, np.ones(256, np.float32))
    expect = np.array([[a * b for b in range(-128, 128)] for a in range(-128, 128)], np.int64)
    assert np.array_equal(acc.astype(np.int64), expect)


def test_int4_decode_exhaustive():
    """Every packed byte against every activation in [-127, 127], at both nibble positions."""
    w4 = np.arange(256, dtype=np.uint8).reshape(256, 1)  # N=256 rows, K=2
    qs = np.arange(-127, 128, dtype=np.int64)
    q = np.zeros((2 * qs.size, 2), np.int8)
    q[: qs.size, 0] = qs       # activation on the even k (low nibble)
    q[qs.size:, 1] = qs        # activation on the odd k (high nibble)
    _, acc = oracle.gemm_w4a8(q, np.ones(q.shape[0], np.float32), w4, np.ones(256, np.float32))
    dec = _decode_w4_brute(w4, 2)
    expect = np.concatenate([np.outer(qs, dec[:, 0]), np.outer(qs, dec[:, 1])])
    assert np.array_equal(acc.astype(np.int64), expect)


@pytest.mark.parametrize("c", [1, 127, -127, -128])
def test_identity_weights(c):
    r = _rng(20)
    K = 48
    q = r.integers(-127, 128, (6, K), dtype=np.int8)
    w = (np.eye(K, dtype=np.int64) * c).astype(np.int8)
    _, acc = oracle.gemm_w8a8(q, np.ones(6, np.float32), w, np.ones(K, np.float32))
    assert np.array_equal(acc.astype(np.int64), q.astype(np.int64) * c)


@pytest.mark.parametrize("c", [1, 7, -8])
def test_identity_weights_int4(c):
    from exact_int8_gemm_amd.workloads import pack_int4
    r = _rng(21)
    K = 64
    q = r.integers(-127, 128, (5, K), dtype=np.int8)
    w4 = pack_int4(np.eye(K, dtype=np.int64) * c)
    _, acc = oracle.gemm_w4a8(q, np.ones(5, np.float32), w4, np.ones(K, np.float32))
    assert np.array_equal(acc.astype(np.int64), q.astype(np.int64) * c)


def test_linearity_symmetry_zero_permutation_split():
    r = _rng(22)
    M, N, K = 7, 9, 160
    q1 = r.integers(-60, 61, (M, K), dtype=np.int8)
    q2 = r.integers(-60, 61, (M, K), dtype=np.int8)
    w = r.integers(-127, 128, (N, K), dtype=np.int8)
    ones_m, ones_n = np.ones(M, np.float32), np.ones(N, np.float32)
    a = lambda q, ww=w: oracle.gemm_w8a8(q, ones_m[: q.shape[0]], ww, ones_n[: ww.shape[0]])[1].astype(np.int64)
    # linear in q
    assert np.array_equal(a((q1 + q2).astype(np.int8)), a(q1) + a(q2))
    # odd symmetry
    assert np.array_equal(a((-q1).astype(np.int8)), -a(q1))
    # zero
    assert not a(np.zeros_like(q1)).any()
    # a common permutation of k leaves every sum unchanged
    perm = r.permutation(K)
    assert np.array_equal(a(q1[:, perm].copy(), w[:, perm].copy()), a(q1))
    # split of k into two ranges adds up (the basis of an exact split-K)
    k1 = 96
    left = a(q1[:, :k1].copy(), w[:, :k1].copy())
    right = a(q1[:, k1:].copy(), w[:, k1:].copy())
    assert np.array_equal(left + right, a(q1))
    # a row permutation of q permutes the rows of the result: rows are independent
    rp = r.permutation(M)
    assert np.array_equal(a(q1[rp].copy()), a(q1)[rp])
    # linear in w
    w2 = r.integers(-60, 61, (N, K), dtype=np.int8)
    w3 = r.integers(-60, 61, (N, K), dtype=np.int8)
    assert np.array_equal(a(q1, (w2 + w3).astype(np.int8)), a(q1, w2) + a(q1, w3))


def test_extreme_sums_and_int32_bound():
    # the largest-magnitude sums that still fit: K * 128 * 128 < 2^31 for K = 131040
    K = 131040
    q = np.full((2, K), -128, np.int8)
    q[1] = 127
    w = np.full((2, K), -128, np.int8)
    w[1] = 127
    _, acc = oracle.gemm_w8a8(q, np.ones(2, np.float32), w, np.ones(2, np.float32))
    assert acc.astype(np.int64).tolist() == [[K * 16384, -K * 16256], [-K * 16256, K * 16129]]
    # one past the int32 range is reported, not wrapped
    K2 = 131072
    with pytest.raises(oracle.OracleError):
        oracle.gemm_w8a8(np.full((1, K2), -128, np.int8), np.ones(1, np.float32),
                         np.full((1, K2), -128, np.int8), np.ones(1, np.float32))


# ------------------------------------------------------------------ quantizer

def _check_row_exact(x, q, s):
    """s must be the correctly rounded amax/127 and q the clamped half-even rint of
    the correctly rounded x/s (or the R2 special cases)."""
    xf = [float(v) for v in x]
    if not all(math.isfinite(v) for v in xf):
        assert math.isnan(float(s)) and not q.any()
        return
    amax = max(abs(Fraction(v)) for v in xf)
    s_exp = round_f32(amax / 127)
    assert bits(s) == bits(s_exp), (s, s_exp)
    if s_exp == 0:
        assert not q.any()
        return
    sf = frac(s_exp)
    for xv, qv in zip(xf, q):
        t = round_f32(Fraction(xv) / sf)
        r = rint_half_even(frac(t))
        assert int(qv) == max(-127, min(127, r)), (xv, qv, r)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_quantizer_exact_rationals(seed):
    r = _rng(100 + seed)
    x = r.standard_normal((6, 96), dtype=np.float32)
    x[1] *= np.float32(1e-30)    # tiny row (still normal)
    x[2] *= np.float32(3e30)     # huge row
    x[3, 5] = np.float32(40.0)   # one outlier dominates the row
    x[4] = np.float32(1e-44) * np.sign(x[4])  # subnormal amax: scale underflows to 0
    # subnormal scale with lost precision: x/s reaches beyond +-127 and the clamp binds
    x[5] = (np.arange(96) - 60).astype(np.float32) * np.float32(3.0) * np.float32(2.0 ** -149)
    q, s = oracle.quantize_rows(x)
    for m in range(x.shape[0]):
        _check_row_exact(x[m], q[m], s[m])


def test_quantizer_scale_exact_many_magnitudes():
    """s = amax / 127 correctly rounded, over amax spread across the binary32 range."""
    r = _rng(8)
    a = (r.uniform(1.0, 2.0, 4000) * 2.0 ** r.integers(-140, 120, 4000)).astype(np.float32)
    x = np.stack([a, -a * np.float32(0.5)], axis=1)
    q, s = oracle.quantize_rows(x)
    for i in range(a.size):
        assert bits(s[i]) == bits(round_f32(frac(a[i]) / 127)), a[i]


def test_quantizer_properties():
    r = _rng(7)
    x = r.standard_normal((16, 200), dtype=np.float32)
    q, s = oracle.quantize_rows(x)
    # the largest |x| of each row maps to +-127
    idx = np.abs(x).argmax(axis=1)
    assert np.array_equal(np.abs(q[np.arange(16), idx]), np.full(16, 127))
    assert np.abs(q.astype(np.int32)).max() <= 127
    # odd symmetry
    qn, sn = oracle.quantize_rows(-x)
    assert np.array_equal(qn, -q) and np.array_equal(bits(sn), bits(s))
    # power-of-two scaling: same codes, scale times 2^j
    for j in (-20, -3, 1, 7, 40):
        qj, sj = oracle.quantize_rows(x * np.float32(2.0 ** j))
        assert np.array_equal(qj, q)
        assert np.array_equal(bits(sj), bits(s * np.float32(2.0 ** j)))
    # rows are independent: a row's codes do not depend on the others
    q1, s1 = oracle.quantize_rows(x[5:6])
    assert np.array_equal(q1[0], q[5]) and bits(s1)[0] == bits(s)[5]


def test_quantizer_special_rows_are_local():
    x = np.array([[1.0, 2.0, -3.0], [np.nan, 1.0, 0.0], [0.0, 0.0, 0.0], [1.0, -np.inf, 2.0], [4.0, 5.0, 6.0]],
                 np.float32)
    q, s = oracle.quantize_rows(x)
    assert np.isnan(s[1]) and np.isnan(s[3]) and s[2] == 0.0
    assert not q[1].any() and not q[2].any() and not q[3].any()
    qa, sa = oracle.quantize_rows(x[[0, 4]])
    assert np.array_equal(qa, q[[0, 4]]) and np.array_equal(bits(sa), bits(s[[0, 4]]))


def test_static_quantizer_exact_rationals():
    """Static scale: q = clamp(rint(x / s)) with x / s correctly rounded, s copied to every row."""
    r = _rng(120)
    x = r.standard_normal((5, 160), dtype=np.float32)
    x[1] *= np.float32(50.0)           # many values beyond the calibrated range: the clamp binds
    x[2] *= np.float32(1e-3)           # most codes small, many ties near zero
    x[3, ::7] = np.float32(2.5) * np.float32(0.0625)   # exact ties at half-integers of x / s
    for scale in (np.float32(0.0625), np.float32(0.0170001), np.float32(0.0123), np.float32(3.0e-3),
                  np.float32(2.0 ** -140)):
        # last row: values next to (n + 1/2) * s, where x / s sits at a rounding tie and a
        # quotient off by one ulp (e.g. x * (1 / s)) changes the code
        n = np.arange(-80, 80)
        t = ((n + 0.5) * scale).astype(np.float32)
        x[4] = np.where(n % 2 == 0, t, np.nextafter(t, np.float32(np.inf) * np.sign(n + 0.5)))
        q, s = oracle.quantize_rows_static(x, float(scale))
        assert np.array_equal(bits(s), np.full(5, bits(np.float32(scale))))
        for m in range(x.shape[0]):
            for xv, qv in zip(x[m], q[m]):
                t = round_f32(frac(xv) / frac(scale))
                if np.isinf(t):
                    ref = 127 if t > 0 else -127
                else:
                    ref = max(-127, min(127, rint_half_even(frac(t))))
                assert int(qv) == ref, (scale, xv, qv, ref)


def test_static_quantizer_hand_table():
    x = np.array([[0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, 127.5],
                  [1e30, -1e30, np.inf, -np.inf, 200.0, -200.0, 0.0, -0.0],
                  [1.0, np.nan, 2.0, 3.0, 4.0, 5.0, 6.0, 7.0],
                  [0.0] * 8], np.float32)
    q, s = oracle.quantize_rows_static(x, 1.0)
    assert q[0].tolist() == [0, 2, 2, 0, -2, -2, 126, 127]
    assert q[1].tolist() == [127, -127, 127, -127, 127, -127, 0, 0]
    assert np.isnan(s[2]) and not q[2].any()
    assert not q[3].any() and s[3] == 1.0 and s[0] == 1.0 and s[1] == 1.0
    # rows are independent
    qa, sa = oracle.quantize_rows_static(x[[0, 1, 3]], 1.0)
    assert np.array_equal(qa, q[[0, 1, 3]]) and np.array_equal(bits(sa), bits(s[[0, 1, 3]]))


def test_static_quantizer_equals_dynamic_at_row_absmax():
    """With s = amax / 127 of a finite row, the static and the dynamic quantizer agree bit for bit."""
    r = _rng(121)
    x = r.standard_normal((8, 200), dtype=np.float32) * np.float32(3.0)
    qd, sd = oracle.quantize_rows(x)
    for m in range(x.shape[0]):
        qs, ss = oracle.quantize_rows_static(x[m:m + 1], float(sd[m]))
        assert np.array_equal(qs[0], qd[m]) and bits(ss)[0] == bits(sd)[m]


@pytest.mark.parametrize("bad", [0.0, -1.0, float("inf"), float("nan")])
def test_static_quantizer_rejects_bad_scale(bad):
    with pytest.raises(oracle.OracleError):
        oracle.quantize_rows_static(np.ones((1, 4), np.float32), bad)


# ------------------------------------------------------------------ Q8_0 blocks

def _pack_q8_0(w, d_values):
    """Q8_0 bytes from the format's definition, with Python's struct (binary16 'e', little-endian)."""
    import struct
    N, K = w.shape
    out = bytearray()
    for n in range(N):
        for b in range(K // 32):
            out += struct.pack("<e", float(d_values[n, b]))
            out += struct.pack("<32b", *[int(v) for v in w[n, 32 * b:32 * b + 32]])
    return np.frombuffer(bytes(out), np.uint8)


def test_q8_0_hand_fixture():
    # two rows of one block each: scale 1.0 (bits 0x3c00) and -2.0 (0xc000), codes written out
    codes0 = [-128, -1, 0, 1, 127] + [5] * 27
    codes1 = list(range(-16, 16))
    raw = bytes([0x00, 0x3C]) + bytes(c & 0xFF for c in codes0) + bytes([0x00, 0xC0]) + bytes(c & 0xFF for c in codes1)
    w, d = oracle.repack_q8_0(np.frombuffer(raw, np.uint8), 2, 32)
    assert d.tolist() == [[0x3C00], [0xC000]]
    assert w[0].tolist() == codes0 and w[1].tolist() == codes1


def test_q8_0_round_trip_with_struct_packer():
    r = _rng(130)
    N, K = 5, 192
    w = r.integers(-128, 128, (N, K), dtype=np.int8)
    dv = (r.standard_normal((N, K // 32)) * 0.01).astype(np.float16)
    dv[0, 0] = np.float16(6.0e-8)      # subnormal binary16
    dv[1, 2] = np.float16(-0.0)
    blocks = _pack_q8_0(w, dv)
    assert blocks.size == N * (K // 32) * 34
    w2, d2 = oracle.repack_q8_0(blocks, N, K)
    assert np.array_equal(w2, w)
    assert np.array_equal(d2, dv.view(np.uint16))


# ------------------------------------------------------------------ Q4_K blocks

def _pack_q4_k(codes, d16, dmin16, sc, mn):
    """Q4_K super-blocks from the layout's description (not from the oracle's unpacking):
    d, dmin little-endian binary16; 12 scale bytes holding 6-bit sc_j / m_j (j < 4 in the low
    6 bits of bytes j and j + 4; j >= 4 as a low nibble pair in byte j + 4 plus the top 2 bits
    of bytes j - 4 and j); 128 code bytes, byte 32 g + l = code[64 g + l] | code[64 g + 32 + l] << 4."""
    import struct
    N, K = codes.shape
    out = bytearray()
    for n in range(N):
        for t in range(K // 256):
            s = [0] * 12
            for j in range(8):
                c, m = int(sc[n, 8 * t + j]), int(mn[n, 8 * t + j])
                if j < 4:
                    s[j] |= c & 63
                    s[j + 4] |= m & 63
                else:
                    s[j + 4] |= (c & 15) | ((m & 15) << 4)
                    s[j - 4] |= (c >> 4) << 6
                    s[j] |= (m >> 4) << 6
            blk = codes[n, 256 * t:256 * t + 256].astype(np.int64)
            qs = [0] * 128
            for g in range(4):
                for l in range(32):
                    qs[32 * g + l] = int(blk[64 * g + l]) | (int(blk[64 * g + 32 + l]) << 4)
            out += struct.pack("<e", float(d16[n, t])) + struct.pack("<e", float(dmin16[n, t]))
            out += bytes(s) + bytes(qs)
    return np.frombuffer(bytes(out), np.uint8)


def _q4k_case(seed, N, K, zero_mins=False):
    r = _rng(seed)
    codes = r.integers(0, 16, (N, K), dtype=np.int8)
    d16 = (r.uniform(0.5, 1.0, (N, K // 256)) * 2.0 ** r.integers(-14, -4, (N, K // 256))).astype(np.float16)
    dmin16 = (r.uniform(0.5, 1.0, (N, K // 256)) * 2.0 ** r.integers(-14, -4, (N, K // 256))).astype(np.float16)
    sc = r.integers(0, 64, (N, K // 32))
    mn = np.zeros((N, K // 32), np.int64) if zero_mins else r.integers(0, 64, (N, K // 32))
    return codes, d16, dmin16, sc, mn


def test_q4_k_hand_fixture():
    """One super-block written by hand; the repack only splits its bytes: the 16 leading
    bytes (d, dmin, scales) go to the header plane, the 128 code bytes to the codes plane."""
    s = [0] * 12
    s[0] = 0b11000001     # sc0 = 1, top bits = high bits of sc4
    s[4] = 0b01000010     # m0 = 2, top bits = high bits of m4
    s[8] = 0x5A           # sc4 low nibble 0xA, m4 low nibble 0x5
    qs = [0] * 128
    qs[0] = 0x73          # weight 0: code 3; weight 32: code 7
    qs[32 + 5] = 0xF0     # weight 64 + 5: code 0; weight 96 + 5: code 15
    raw = bytes([0x00, 0x3C, 0x00, 0x38]) + bytes(s) + bytes(qs)   # d = 1.0, dmin = 0.5
    two = raw + bytes(range(144))   # a second super-block of the same row: K = 512
    w4, hdr = oracle.repack_q4_k(np.frombuffer(two, np.uint8), 1, 512)
    assert hdr.shape == (1, 2, 16) and w4.shape == (1, 256)
    assert bytes(hdr[0, 0]) == raw[:16] and bytes(hdr[0, 1]) == bytes(range(16))
    assert w4[0, 0] == 0x73 and w4[0, 37] == 0xF0 and int(w4[0, :128].sum()) == 0x73 + 0xF0
    assert bytes(w4[0, 128:]) == bytes(range(16, 144))


def test_q4_k_round_trip_with_independent_packer():
    """Blocks packed from the layout's description; putting the header and code planes back
    together (numpy slicing) gives the blocks again, byte for byte."""
    codes, d16, dmin16, sc, mn = _q4k_case(140, 3, 512)
    d16[0, 0] = np.float16(6.0e-8)     # subnormal binary16 scale
    blocks = _pack_q4_k(codes, d16, dmin16, sc, mn)
    w4, hdr = oracle.repack_q4_k(blocks, 3, 512)
    again = np.concatenate([hdr, w4.reshape(3, 2, 128)], axis=2).reshape(-1)
    assert np.array_equal(again, blocks)
    # the code plane keeps the file's nibble order: byte 32 g + l of a super-block holds
    # the code of weight 64 g + l (low nibble) and of weight 64 g + 32 + l (high nibble)
    for n in range(3):
        for t in range(2):
            qs = w4[n, 128 * t:128 * t + 128].astype(np.int64)
            for g in range(4):
                assert np.array_equal(qs[32 * g:32 * g + 32] & 15, codes[n, 256 * t + 64 * g:256 * t + 64 * g + 32])
                assert np.array_equal(qs[32 * g:32 * g + 32] >> 4, codes[n, 256 * t + 64 * g + 32:256 * t + 64 * g + 64])


def test_q4_k_gemm_within_bound_of_exact_dot_product():
    """|y - s_a * sum_k w_k a_k| stays within the rounding bound of the fp32 chain (exact sum in fp64)."""
    N, K, M = 6, 1024, 4
    codes, d16, dmin16, sc, mn = _q4k_case(141, N, K)
    blocks = _pack_q4_k(codes, d16, dmin16, sc, mn)
    r = _rng(142)
    q = r.integers(-127, 128, (M, K), dtype=np.int8)
    s_a = r.uniform(1e-3, 1e-2, M).astype(np.float32)
    y = oracle.gemm_w4a8_q4k(q, s_a, blocks, N)
    dd = np.repeat(np.repeat(d16.astype(np.float64), 8, axis=1) * sc, 32, axis=1)     # d * sc per weight
    dm = np.repeat(np.repeat(dmin16.astype(np.float64), 8, axis=1) * mn, 32, axis=1)  # dmin * m per weight
    wv = dd * codes - dm                                                                 # exact in fp64
    for m in range(M):
        a = q[m].astype(np.float64)
        exact = (wv * a).sum(axis=1)
        mag = (np.abs(dd * codes) * np.abs(a)).sum(axis=1) + (np.abs(dm) * np.abs(a)).sum(axis=1)
        bound = 2 * (K // 32) * 2.0 ** -24 * mag + 2.0 ** -23 * np.abs(exact)
        assert (np.abs(y[m] / s_a[m].astype(np.float64) - exact) <= bound + 1e-30).all(), m


def _q4k_replay(codes, d16, dmin16, sc, mn, q, s_a, m, n, order="scale_then_min"):
    """The fixed fp32 chain of one output, replayed in exact rationals with binary32 rounding
    after every fused step: per 32-weight sub-block b in ascending k, P = sum code * a and
    S = sum a (Python integers), D = d * sc and Mn = dmin * m (exact), then
    f = rn(P D + f) and f = rn(-S Mn + f); finally y = rn(f s_a)."""
    K = codes.shape[1]
    f = np.float32(0.0)
    for b in range(K // 32):
        t = b // 8
        P = sum(int(codes[n, k]) * int(q[m, k]) for k in range(32 * b, 32 * b + 32))
        S = sum(int(q[m, k]) for k in range(32 * b, 32 * b + 32))
        D = Fraction(float(d16[n, t])) * int(sc[n, b])
        Mn = Fraction(float(dmin16[n, t])) * int(mn[n, b])
        if order == "scale_then_min":
            f = round_f32(Fraction(P) * D + frac(f))
            f = round_f32(Fraction(-S) * Mn + frac(f))
        else:   # the other order, used only to find inputs where the two differ
            f = round_f32(Fraction(-S) * Mn + frac(f))
            f = round_f32(Fraction(P) * D + frac(f))
    return round_f32(frac(f) * frac(s_a[m]))


@pytest.mark.parametrize("seed", [0, 1])
def test_q4_k_gemm_exact_rationals(seed):
    """Every output of the Q4_K GEMM equals the exact-rational replay of its fp32 chain
    (scale term, then min term, per sub-block, ascending; one rounding per fused step)."""
    N, K, M = 3, 512, 3
    codes, d16, dmin16, sc, mn = _q4k_case(150 + seed, N, K)
    blocks = _pack_q4_k(codes, d16, dmin16, sc, mn)
    r = _rng(152 + seed)
    q = r.integers(-127, 128, (M, K), dtype=np.int8)
    s_a = r.uniform(1e-3, 1.0, M).astype(np.float32)
    y = oracle.gemm_w4a8_q4k(q, s_a, blocks, N)
    for m in range(M):
        for n in range(N):
            assert bits(y[m, n]) == bits(_q4k_replay(codes, d16, dmin16, sc, mn, q, s_a, m, n)), (m, n)


def test_q4_k_fold_order_where_orders_differ():
    """Hand-built two-sub-block rows where 'scale term, then min term' and the reverse order
    (or an unfused min term) round to different floats: the oracle must give the first."""
    r = _rng(160)
    found = 0
    for _ in range(4000):
        codes = np.zeros((1, 256), np.int8)
        q = np.zeros((1, 256), np.int8)
        # sub-blocks 0 and 1 carry one nonzero code/activation pair each, plus a few
        # activations on zero codes so that S differs from the code-weighted sum
        for b in (0, 1):
            codes[0, 32 * b] = r.integers(1, 16)
            q[0, 32 * b] = r.integers(-127, 128)
            q[0, 32 * b + 1:32 * b + 4] = r.integers(-127, 128, 3)
        d16 = np.array([[np.float16(r.uniform(0.5, 1.0) * 2.0 ** int(r.integers(-12, -6)))]])
        dmin16 = np.array([[np.float16(r.uniform(0.5, 1.0) * 2.0 ** int(r.integers(-12, -6)))]])
        sc = np.zeros((1, 8), np.int64)
        mn = np.zeros((1, 8), np.int64)
        sc[0, :2] = r.integers(1, 64, 2)
        mn[0, :2] = r.integers(1, 64, 2)
        s_a = np.ones(1, np.float32)
        want = _q4k_replay(codes, d16, dmin16, sc, mn, q, s_a, 0, 0)
        other = _q4k_replay(codes, d16, dmin16, sc, mn, q, s_a, 0, 0, order="min_then_scale")
        # the min term as a rounded product followed by a rounded add
        f = np.float32(0.0)
        for b in (0, 1):
            P = int(codes[0, 32 * b]) * int(q[0, 32 * b])
            S = sum(int(v) for v in q[0, 32 * b:32 * b + 32])
            D = Fraction(float(d16[0, 0])) * int(sc[0, b])
            Mn = Fraction(float(dmin16[0, 0])) * int(mn[0, b])
            f = round_f32(Fraction(P) * D + frac(f))
            f = round_f32(frac(round_f32(Fraction(-S) * Mn)) + frac(f))
        unfused = round_f32(frac(f))
        if bits(want) == bits(other) and bits(want) == bits(unfused):
            continue
        y = oracle.gemm_w4a8_q4k(q, s_a, _pack_q4_k(codes, d16, dmin16, sc, mn), 1)
        assert bits(y[0, 0]) == bits(want)
        found += 1
        if found == 20:
            break
    assert found == 20


def test_q4_k_gemm_without_mins_is_the_block_scale_gemm():
    """Zero mins and d * sc exact in binary16: the Q4_K path is the pinned block-scale path, bit for bit."""
    N, K, M = 5, 512, 3
    codes, _, dmin16, sc, mn = _q4k_case(143, N, K, zero_mins=True)
    d16 = np.full((N, K // 256), np.float16(2.0 ** -10))
    blocks = _pack_q4_k(codes, d16, dmin16, sc, mn)
    r = _rng(144)
    q = r.integers(-127, 128, (M, K), dtype=np.int8)
    s_a = r.uniform(1e-3, 1e-2, M).astype(np.float32)
    y = oracle.gemm_w4a8_q4k(q, s_a, blocks, N)
    dbits = (np.float64(2.0 ** -10) * sc).astype(np.float16).view(np.uint16)   # exact: sc < 64
    y_b, _ = oracle.gemm_w8a8_blockscale(q, s_a, codes, dbits)
    assert np.array_equal(bits(y), bits(y_b))


# ------------------------------------------------------------------ epilogues

def test_channel_epilogue_exact_rationals():
    r = _rng(30)
    M, N, K = 9, 11, 64
    q = r.integers(-127, 128, (M, K), dtype=np.int8)
    w = r.integers(-127, 128, (N, K), dtype=np.int8)
    s_a = r.uniform(1e-3, 1.0, M).astype(np.float32)
    s_a[0] = np.float32(1e-41)  # subnormal products must not be flushed
    s_w = r.uniform(1e-3, 1e-2, N).astype(np.float32)
    y, acc = oracle.gemm_w8a8(q, s_a, w, s_w)
    for m in range(M):
        for n in range(N):
            t = round_f32(Fraction(int(acc[m, n])) * frac(s_a[m]))
            e = round_f32(frac(t) * frac(s_w[n]))
            assert bits(y[m, n]) == bits(e)


def test_channel_epilogue_large_acc_rounds_to_nearest_even():
    # acc above 2^24 is not representable; (float)acc must round half to even
    K = 131040
    q = np.full((1, K), 127, np.int8)
    w = np.full((3, K), 127, np.int8)
    w[1, :5] = 126   # acc = K*16129 - 5*127
    w[2, :1] = 0     # acc = K*16129 - 16129
    y, acc = oracle.gemm_w8a8(q, np.ones(1, np.float32), w, np.ones(3, np.float32))
    for n in range(3):
        assert bits(y[0, n]) == bits(round_f32(Fraction(int(acc[0, n]))))
    assert int(acc[0, 0]) == K * 16129


def test_w4a8_epilogue_exact_rationals():
    r = _rng(31)
    M, N, K = 4, 7, 64
    q = r.integers(-127, 128, (M, K), dtype=np.int8)
    w4 = r.integers(0, 256, (N, K // 2), dtype=np.uint8)
    s_a = r.uniform(1e-3, 1.0, M).astype(np.float32)
    s_w = r.uniform(1e-3, 1e-2, N).astype(np.float32)
    y, acc = oracle.gemm_w4a8(q, s_a, w4, s_w)
    ref = _brute_acc(q, _decode_w4_brute(w4, K))
    for m in range(M):
        for n in range(N):
            t = round_f32(Fraction(int(ref[m, n])) * frac(s_a[m]))
            assert bits(y[m, n]) == bits(round_f32(frac(t) * frac(s_w[n])))


def test_f16_to_f32_exhaustive_vs_numpy():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.f16_to_f32(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(bits(got)[~nan], bits(ref)[~nan])


@pytest.mark.parametrize("seed", [0, 1])
def test_blockscale_exact_rationals(seed):
    """Partials by brute force, the ascending fused combine in exact rationals."""
    from exact_int8_gemm_amd.workloads import block_scale_bits
    r = _rng(40 + seed)
    M, N, K = 3, 5, 160
    q = r.integers(-127, 128, (M, K), dtype=np.int8)
    w = r.integers(-127, 128, (N, K), dtype=np.int8)
    d = block_scale_bits(r, N, K // 32)
    d[0, 1] = 0x8001   # negative subnormal scale
    d[1, 0] = 0x0000   # zero scale
    s_a = r.uniform(1e-3, 1.0, M).astype(np.float32)
    y, part = oracle.gemm_w8a8_blockscale(q, s_a, w, d, want_partials=True)
    dv = d.view(np.float16).astype(np.float64)
    for m in range(M):
        for n in range(N):
            f = np.float32(0.0)
            for b in range(K // 32):
                p = sum(int(q[m, k]) * int(w[n, k]) for k in range(32 * b, 32 * b + 32))
                assert int(part[m, n, b]) == p
                f = round_f32(Fraction(p) * Fraction(float(dv[n, b])) + frac(f))
            assert bits(y[m, n]) == bits(round_f32(frac(f) * frac(s_a[m])))


def test_blockscale_fma_is_fused_not_mul_add():
    """Cases where one fused multiply-add and a rounded multiply followed by a
    rounded add give different floats: the oracle must give the fused one."""
    r = _rng(60)
    found = 0
    for _ in range(20000):
        q0, w0, q1, w1 = (int(v) for v in r.integers(-127, 128, 4))
        d0, d1 = (int(v) for v in r.integers(0x0400, 0x7800, 2))  # positive normal binary16
        f0 = round_f32(Fraction(q0 * w0) * Fraction(float(np.uint16(d0).view(np.float16))))
        p1 = Fraction(q1 * w1) * Fraction(float(np.uint16(d1).view(np.float16)))
        fused = round_f32(p1 + frac(f0))
        two_step = round_f32(frac(round_f32(p1)) + frac(f0))
        if bits(fused) == bits(two_step):
            continue
        q = np.zeros((1, 64), np.int8)
        w = np.zeros((1, 64), np.int8)
        q[0, 0], w[0, 0], q[0, 32], w[0, 32] = q0, w0, q1, w1
        y, _ = oracle.gemm_w8a8_blockscale(q, np.ones(1, np.float32), w, np.array([[d0, d1]], np.uint16))
        assert bits(y[0, 0]) == bits(fused)
        found += 1
        if found == 20:
            break
    assert found == 20


def test_blockscale_partials_sum_to_channel_acc():
    r = _rng(50)
    M, N, K = 6, 7, 256
    q = r.integers(-127, 128, (M, K), dtype=np.int8)
    w = r.integers(-127, 128, (N, K), dtype=np.int8)
    d = np.full((N, K // 32), 0x3C00, np.uint16)   # all block scales 1.0
    y, part = oracle.gemm_w8a8_blockscale(q, np.ones(M, np.float32), w, d, want_partials=True)
    _, acc = oracle.gemm_w8a8(q, np.ones(M, np.float32), w, np.ones(N, np.float32))
    assert np.array_equal(part.astype(np.int64).sum(axis=2), acc.astype(np.int64))
    # with unit scales and |running sum| < 2^24 every fma is exact: y = acc
    assert np.array_equal(y, acc.astype(np.float32))


# --------------------------------------------------------------- hand cases

def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _fl(v):
    return float(v) if not isinstance(v, str) else float(v.replace("inf", "inf"))


def test_golden_quantize():
    for case in _golden()["quantize"]:
        x = np.array([[_fl(v) for v in case["x"]]], np.float32)
        q, s = oracle.quantize_rows(x)
        assert q[0].tolist() == case["q"], case["why"]
        se = _fl(case["s"])
        assert (math.isnan(s[0]) and math.isnan(se)) or s[0] == se, case["why"]


def test_golden_gemms():
    g = _golden()
    c = g["gemm_w8a8"]
    y, acc = oracle.gemm_w8a8(np.array(c["q"], np.int8), np.array(c["s_a"], np.float32),
                              np.array(c["w"], np.int8), np.array(c["s_w"], np.float32))
    assert acc.tolist() == c["acc"] and y.tolist() == c["y"]
    c = g["gemm_w4a8"]
    y, acc = oracle.gemm_w4a8(np.array(c["q"], np.int8), np.array(c["s_a"], np.float32),
                              np.array(c["w4"], np.uint8), np.array(c["s_w"], np.float32))
    assert acc.tolist() == c["acc"] and y.tolist() == c["y"]
    c = g["gemm_w8a8_blockscale"]
    q = np.ones((1, 64), np.int8)
    w = np.concatenate([np.ones(32), 2 * np.ones(32)]).astype(np.int8).reshape(1, 64)
    y, part = oracle.gemm_w8a8_blockscale(q, np.array(c["s_a"], np.float32), w,
                                          np.array([c["d_bits"]], np.uint16), want_partials=True)
    assert part[0, 0].tolist() == c["partials"] and float(y[0, 0]) == c["y"]
    c = g["gemm_w8a8_blockscale_subnormal"]
    y, part = oracle.gemm_w8a8_blockscale(np.ones((1, 32), np.int8), np.array(c["s_a"], np.float32),
                                          np.ones((1, 32), np.int8), np.array([c["d_bits"]], np.uint16),
                                          want_partials=True)
    assert part[0, 0].tolist() == c["partials"] and float(y[0, 0]) == c["y"]


def test_pack_int4_known_bytes():
    from exact_int8_gemm_amd.workloads import pack_int4
    assert pack_int4(np.array([[1, -1, 7, -8]])).tolist() == [[0xF1, 0x87]]
    assert pack_int4(np.array([[0, 0, -1, -1]])).tolist() == [[0x00, 0xFF]]
