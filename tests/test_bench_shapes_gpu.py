"""GPU parity at the full sizes of the extra workloads that bench.py times
(W4A8 prefill, block-scale decode, Q4_K), on the same inputs, against the
CPU oracle.

Rows are independent in the definition, so the oracle run on a subset of
rows gives exactly those rows' outputs; at M > 16 the checks use sampled
rows (the first and last rows of tiles among them).
"""
import numpy as np
import pytest
import torch

import oracle
from exact_int8_gemm_amd import prism
from exact_int8_gemm_amd import workloads as wl
from gpu_util import DEV, assert_same_floats, assert_same_ints, dev, host

pytestmark = pytest.mark.gpu


def _rows(M, seed):
    fixed = [r for r in (0, 1, 127, 128, 255, 256, M - 1) if r < M]
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([fixed, rng.choice(M, min(M, 17), replace=False)])).astype(np.int64)


def _quantize_both(x):
    q_ref, s_ref = oracle.quantize_rows(x)
    q, s = prism.quantize_rows(dev(x))
    torch.cuda.synchronize()
    assert_same_floats(host(s), s_ref, "scale")
    assert_same_ints(host(q), q_ref, "codes")
    return q, s, q_ref, s_ref


@pytest.mark.parametrize("M", [512, 2048])
def test_w4a8_prefill_full_size_sampled_rows(M):
    """N = 12288, K = 4096 (the W4A8 weights), M > 64: the 4-bit tiled path,
    with the 64 seeded rows repeated as in the benchmark."""
    c = wl.w4()
    x = c["x"][[i % 64 for i in range(M)]]
    q, s, q_ref, s_ref = _quantize_both(x)
    N = c["w4"].shape[0]
    acc = torch.empty((M, N), dtype=torch.int32, device=DEV)
    y = host(prism.gemm_w4a8(q, s, dev(c["w4"]), dev(c["s_w"]), acc=acc))
    rows = _rows(M, M)
    y_ref, acc_ref = oracle.gemm_w4a8(q_ref[rows], s_ref[rows], c["w4"], c["s_w"])
    assert_same_ints(host(acc)[rows], acc_ref, "acc sampled rows")
    assert_same_floats(y[rows], y_ref, "y sampled rows")


@pytest.mark.parametrize("M", [1, 4, 16])
def test_block_scale_decode_full_size(M):
    """N = 17408, K = 5120 with fp16 block scales, M <= 16: the per-wave kernel (M = 1, 4)
    and the small-M block kernel (M = 16), every row against the oracle."""
    c = wl.block()
    q, s, q_ref, s_ref = _quantize_both(c["x"][:M].copy())
    y = host(prism.gemm_w8a8_blockscale(q, s, dev(c["w"]), dev(c["d"])))
    y_ref, _ = oracle.gemm_w8a8_blockscale(q_ref, s_ref, c["w"], c["d"])
    assert_same_floats(y, y_ref, "y")


def _q4k_blocks(seed, N, K):
    """Random Q4_K super-block bytes (144 per 256 weights) whose d and dmin are
    finite binary16 values in [2^-14, 2^-5): every scale, min and code pattern
    occurs, and no output is NaN or infinite."""
    rng = np.random.default_rng(seed)
    nsb = N * (K // 256)
    blocks = rng.integers(0, 256, (nsb, 144), dtype=np.uint8)
    dd = (rng.uniform(0.5, 1.0, (nsb, 2)) * 2.0 ** rng.integers(-13, -5, (nsb, 2))).astype("<f2")
    blocks[:, 0:4] = dd.view(np.uint8).reshape(nsb, 4)
    return blocks.reshape(-1)


@pytest.mark.parametrize("M", [1, 4, 2048])
def test_q4k_full_size(M):
    """Q4_K weights of the block-scale shape (17408 x 5120): the repacked
    planes in full, and the GEMM (M = 1: small-M block kernel, every output;
    M = 2048: tiled kernel, sampled rows)."""
    N, K = 17408, 5120
    blocks = _q4k_blocks(12, N, K)
    w4, hdr = prism.repack_q4_k(dev(blocks), N, K)
    if M == 1:
        w_ref, h_ref = oracle.repack_q4_k(blocks, N, K)
        torch.cuda.synchronize()
        assert_same_ints(host(w4), w_ref, "packed codes")
        assert_same_ints(host(hdr), h_ref, "headers")
    q, s, q_ref, s_ref = _quantize_both(wl.block()["x"][:M].copy())
    y = host(prism.gemm_w4a8_q4k(q, s, w4, hdr))
    rows = _rows(M, 7) if M > 16 else np.arange(M)
    y_ref = oracle.gemm_w4a8_q4k(q_ref[rows], s_ref[rows], blocks, N)
    assert np.isfinite(y_ref).all()
    assert_same_floats(y[rows], y_ref, "y")


def test_block_scale_large_tiles_ragged():
    """Block-scale with enough 128 x 128 tiles for the eight-wave tiles (M = 2113, N =
    16416: ragged last row and column tiles) and K = 288 (a last stage of one block):
    sampled rows, every column, against the oracle."""
    M, N, K = 2113, 16416, 288
    rng = np.random.default_rng(31)
    q = rng.integers(-128, 128, (M, K), dtype=np.int8)
    s_a = rng.uniform(1e-3, 1e-1, M).astype(np.float32)
    w = rng.integers(-128, 128, (N, K), dtype=np.int8)
    d = rng.uniform(1e-4, 1e-2, (N, K // 32)).astype(np.float16).view(np.uint16)
    y = host(prism.gemm_w8a8_blockscale(dev(q), dev(s_a), dev(w), dev(d)))
    rows = _rows(M, 3)
    y_ref, _ = oracle.gemm_w8a8_blockscale(q[rows], s_a[rows], w, d)
    assert_same_floats(y[rows], y_ref, "y sampled rows")


def test_q4k_large_tiles_ragged():
    """Q4_K with enough 128 x 128 tiles for the eight-wave tiles (M = 1100, N = 16400:
    ragged last tiles): sampled rows, every column, against the oracle."""
    M, N, K = 1100, 16400, 256
    blocks = _q4k_blocks(33, N, K)
    w4, hdr = prism.repack_q4_k(dev(blocks), N, K)
    x = np.random.default_rng(34).standard_normal((M, K), dtype=np.float32)
    q, s, q_ref, s_ref = _quantize_both(x)
    y = host(prism.gemm_w4a8_q4k(q, s, w4, hdr))
    rows = _rows(M, 5)
    y_ref = oracle.gemm_w4a8_q4k(q_ref[rows], s_ref[rows], blocks, N)
    assert_same_floats(y[rows], y_ref, "y sampled rows")
