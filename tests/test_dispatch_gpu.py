"""Every entry of the W8A8 / W4A8 dispatch table gives the same bits (GPU).

The plain calls pick a kernel, a tile shape and a K split from (M, N, K).
That choice may vary with M only because every entry computes the same exact
int32 sums and the same per-element fp32 epilogue.  Here each applicable
entry is run on its own through the ``*_variant`` calls and compared with the
CPU oracle bit for bit; entries that do not apply must be refused.
"""
import numpy as np
import pytest
import torch

import oracle
from exact_int8_gemm_amd import prism
from exact_int8_gemm_amd import workloads as wl
from gpu_util import DEV, assert_same_floats, assert_same_ints, dev, host

pytestmark = pytest.mark.gpu

SMALL = ["small_1x4", "small_1x8", "small_1x16", "small_2x4", "small_2x8", "small_2x16", "small_3x4", "small_3x8",
         "small_4x4", "small_4x8", "small_balanced"]
TILES8 = ["tile_256x256", "tile_256x192", "tile_256x320", "tile_256x128", "tile_128x128", "tile_128x128_split2",
          "tile_128x128_split3", "tile_128x128_split4", "tile_64x128", "tile_64x128_split2", "tile_64x128_split3",
          "tile_64x128_split4", "tile_128x96", "tile_128x96_split2", "tile_192x128"]
TILES4 = ["tile_256x256", "tile_256x192", "tile_256x320", "tile_128x128", "tile_128x128_split2", "tile_128x128_split3",
          "tile_128x128_split4", "tile_64x128", "tile_64x128_split2", "tile_64x128_split3", "tile_64x128_split4"]


def _inputs(seed, M, N, K, w4=False):
    rng = np.random.default_rng(seed)
    q = rng.integers(-128, 128, (M, K), dtype=np.int8)      # the whole int8 range, -128 included
    s_a = rng.uniform(1e-3, 1e-2, M).astype(np.float32)
    s_w = wl.channel_scales(rng, N)
    if w4:
        w = rng.integers(-8, 8, (N, K), dtype=np.int8)
        return q, s_a, wl.pack_int4(w), s_w
    return q, s_a, wl.int8_weights(rng, N, K), s_w


def _run_all(fn, names, q, s_a, w, s_w, y_ref, acc_ref):
    M, N = y_ref.shape
    for name in names:
        acc = torch.full((M, N), 7, dtype=torch.int32, device=DEV)
        y = torch.full((M, N), 3.0, dtype=torch.float32, device=DEV)
        fn(q, s_a, w, s_w, name, y=y, acc=acc)
        torch.cuda.synchronize()
        assert_same_ints(host(acc), acc_ref, "acc (%s)" % name)
        assert_same_floats(host(y), y_ref, "y (%s)" % name)


@pytest.mark.parametrize("M", [1, 5, 16, 17, 33, 64])
@pytest.mark.parametrize("N,K", [(100, 160), (300, 2064)])
def test_w8a8_every_entry_small_m(M, N, K):
    q, s_a, w, s_w = _inputs(M * 1000 + N + K, M, N, K)
    y_ref, acc_ref = oracle.gemm_w8a8(q, s_a, w, s_w)
    _run_all(prism.gemm_w8a8_variant, ["auto"] + SMALL + TILES8, dev(q), dev(s_a), dev(w), dev(s_w), y_ref, acc_ref)


@pytest.mark.parametrize("M", [65, 129, 300])
@pytest.mark.parametrize("N,K", [(100, 160), (257, 4112)])
def test_w8a8_every_entry_large_m(M, N, K):
    q, s_a, w, s_w = _inputs(M * 1000 + N + K, M, N, K)
    y_ref, acc_ref = oracle.gemm_w8a8(q, s_a, w, s_w)
    qd, sad, wd, swd = dev(q), dev(s_a), dev(w), dev(s_w)
    _run_all(prism.gemm_w8a8_variant, ["auto"] + TILES8, qd, sad, wd, swd, y_ref, acc_ref)
    y = torch.full((M, N), 3.0, dtype=torch.float32, device=DEV)
    for name in SMALL:   # the small-M kernel holds at most 64 rows: refused, nothing written
        with pytest.raises(prism.PrismError):
            prism.gemm_w8a8_variant(qd, sad, wd, swd, name, y=y)
    torch.cuda.synchronize()
    assert (host(y) == 3.0).all()


@pytest.mark.parametrize("M", [1, 16, 33, 64, 65, 200])
@pytest.mark.parametrize("N,K", [(300, 1056), (130, 4128)])
def test_w4a8_every_entry(M, N, K):
    q, s_a, w4, s_w = _inputs(M * 7 + 1, M, N, K, w4=True)
    y_ref, acc_ref = oracle.gemm_w4a8(q, s_a, w4, s_w)
    qd, sad, wd, swd = dev(q), dev(s_a), dev(w4), dev(s_w)
    names = ["auto"] + TILES4 + (SMALL if M <= 64 else [])
    _run_all(prism.gemm_w4a8_variant, names, qd, sad, wd, swd, y_ref, acc_ref)
    for name in [n for n in TILES8 if n not in TILES4]:   # int8-only tiles
        with pytest.raises(prism.PrismError):
            prism.gemm_w4a8_variant(qd, sad, wd, swd, name)


@pytest.mark.parametrize("M,K", [(31, 9728), (32, 7664), (32, 7680), (48, 5104), (48, 5120), (64, 3824), (64, 3840),
                                 (64, 9728)])
def test_w8a8_small_m_or_tiled(M, K):
    """With int8 weights and few columns, 32 <= M <= 64 rows take the tiled
    path (64 x 128 or 128 x 128 tiles, K split by the cost model) once M K >=
    245760, the small-M kernel below that; the plain call must give the oracle's bits on
    both sides of the boundary, and so must every small-M and tiled entry."""
    N = 300
    q, s_a, w, s_w = _inputs(M * 11 + K, M, N, K)
    y_ref, acc_ref = oracle.gemm_w8a8(q, s_a, w, s_w)
    names = ["auto"] + SMALL + [n for n in TILES8 if "128" in n]
    _run_all(prism.gemm_w8a8_variant, names, dev(q), dev(s_a), dev(w), dev(s_w), y_ref, acc_ref)
    y = prism.gemm_w8a8(dev(q), dev(s_a), dev(w), dev(s_w))
    torch.cuda.synchronize()
    assert_same_floats(host(y), y_ref, "y (plain call)")


@pytest.mark.parametrize("w4,M,N,K", [(False, 7, 16400, 256), (False, 8, 16400, 256), (True, 23, 16416, 256),
                                      (True, 24, 16416, 256), (True, 15, 16416, 8192), (True, 16, 16416, 8192),
                                      (False, 23, 2048, 9728), (False, 24, 2048, 9728), (False, 55, 2048, 4096),
                                      (False, 56, 2048, 4096), (True, 47, 1024, 8192), (True, 48, 1024, 8192),
                                      (True, 32, 8192, 16384)])
def test_small_m_or_tiled_boundaries(w4, M, N, K):
    """Up to 64 rows the plain calls choose between the small-M kernel and
    the 64 x 128 tiles from M, N and K (more than 16384 columns: tiles from
    8 int8 rows, 24 4-bit rows or 16 where K >= 8192; otherwise int8 from 24
    rows where M K >= 229376, 4-bit by M K and N K); on both sides of each
    boundary the plain call, one small-M entry and one tile entry must give
    the oracle's bits."""
    q, s_a, w, s_w = _inputs(M * 13 + N + K, M, N, K, w4=w4)
    y_ref, acc_ref = (oracle.gemm_w4a8 if w4 else oracle.gemm_w8a8)(q, s_a, w, s_w)
    fn = prism.gemm_w4a8_variant if w4 else prism.gemm_w8a8_variant
    _run_all(fn, ["auto", "small_2x8", "tile_64x128"], dev(q), dev(s_a), dev(w), dev(s_w), y_ref, acc_ref)
    y = (prism.gemm_w4a8 if w4 else prism.gemm_w8a8)(dev(q), dev(s_a), dev(w), dev(s_w))
    torch.cuda.synchronize()
    assert_same_floats(host(y), y_ref, "y (plain call)")


@pytest.mark.parametrize("M,N", [(2048, 4096), (2048, 4224), (1024, 8192), (1024, 8320)])
def test_w4_tile_family_boundary(M, N):
    """4-bit weights from 65 rows: the plain call keeps 128 x 128 tiles while
    they fit the 512 workgroups that run together (2048 x 4096, 1024 x 8192:
    exactly 512) and weighs the 256-row persistent tiles once there are more
    (4224 and 8320 columns: 528 and 520 tiles, which go to 256 x 192); on both
    sides the plain call and both families must give the oracle's bits."""
    K = 256
    q, s_a, w4, s_w = _inputs(M + N * 7, M, N, K, w4=True)
    y_ref, acc_ref = oracle.gemm_w4a8(q, s_a, w4, s_w)
    _run_all(prism.gemm_w4a8_variant, ["auto", "tile_128x128", "tile_256x192"], dev(q), dev(s_a), dev(w4),
             dev(s_w), y_ref, acc_ref)
    y = prism.gemm_w4a8(dev(q), dev(s_a), dev(w4), dev(s_w))
    torch.cuda.synchronize()
    assert_same_floats(host(y), y_ref, "y (plain call)")


@pytest.mark.parametrize("M,N,K", [(70, 2052, 2080), (129, 1028, 1056), (3, 2560, 4096), (200, 1030, 1056),
                                   (33, 4098, 544)])
def test_k_split_epilogue_rows(M, N, K):
    """A K-split launch finishes in place with its own epilogue kernel: one
    workgroup per 1024 columns of a row when N % 4 == 0 (here 2052, 1028 and
    2560: two or three pieces per row, the last one ragged), a flat walk
    over y otherwise (1030, 4098: runs of four that cross row ends).  Every
    split entry, 4-bit included, must give the oracle's bits and int32 sums."""
    q, s_a, w, s_w = _inputs(M * 3 + N + K, M, N, K)
    y_ref, acc_ref = oracle.gemm_w8a8(q, s_a, w, s_w)
    names = ["auto"] + [n for n in TILES4 if "split" in n]
    _run_all(prism.gemm_w8a8_variant, names, dev(q), dev(s_a), dev(w), dev(s_w), y_ref, acc_ref)
    q, s_a, w4, s_w = _inputs(M * 5 + N + K, M, N, K, w4=True)
    y_ref, acc_ref = oracle.gemm_w4a8(q, s_a, w4, s_w)
    _run_all(prism.gemm_w4a8_variant, names, dev(q), dev(s_a), dev(w4), dev(s_w), y_ref, acc_ref)


@pytest.mark.parametrize("M,N,K", [(600, 1300, 1040), (513, 1100, 4112), (256, 1024, 384), (1030, 2100, 2064)])
def test_w8a8_256_row_tiles_several_column_groups(M, N, K):
    """The 256-row ping-pong tiles (192, 256 and 320 columns) walk each XCD's
    range in groups of four tile columns; shapes with several groups, a short
    last group and ragged M, N and K must give the oracle's bits, also
    through the plain call."""
    q, s_a, w, s_w = _inputs(M + 7 * N + K, M, N, K)
    y_ref, acc_ref = oracle.gemm_w8a8(q, s_a, w, s_w)
    _run_all(prism.gemm_w8a8_variant, ["auto", "tile_256x256", "tile_256x192", "tile_256x320"], dev(q), dev(s_a), dev(w),
             dev(s_w), y_ref, acc_ref)


@pytest.mark.parametrize("w4", [False, True])
@pytest.mark.parametrize("M", [2, 16, 33, 64])
def test_small_m_three_column_blocks(w4, M):
    """N = 9000 has 563 column blocks of 16: the plain call takes workgroups
    of three blocks (one round of 188), the last one ragged; the plain call
    and every small-M entry must give the oracle's bits."""
    N, K = 9000, 1056
    q, s_a, w, s_w = _inputs(M * 31 + (7 if w4 else 0), M, N, K, w4=w4)
    if w4:
        y_ref, acc_ref = oracle.gemm_w4a8(q, s_a, w, s_w)
        fn = prism.gemm_w4a8_variant
    else:
        y_ref, acc_ref = oracle.gemm_w8a8(q, s_a, w, s_w)
        fn = prism.gemm_w8a8_variant
    _run_all(fn, ["auto"] + SMALL, dev(q), dev(s_a), dev(w), dev(s_w), y_ref, acc_ref)


@pytest.mark.parametrize("M,N,K", [(2048, 5120, 5120), (4096, 9728, 2560), (2048, 17408, 5120), (8192, 2560, 9728)])
def test_256_row_tiles_full_size_sampled_rows(M, N, K):
    """The shapes where the plain call picks 256 x 192 or 256 x 320 tiles,
    at full size: the plain call and every 256-row tile width, compared with
    the oracle on sampled rows (rows are independent in the definition, so
    the oracle on a subset of rows gives exactly those rows)."""
    q, s_a, w, s_w = _inputs(M + N + K, M, N, K)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, M // 2, M - 257, M - 256, M - 1],
                                     np.random.default_rng(M + N).choice(M, 16, replace=False)]))
    y_ref, acc_ref = oracle.gemm_w8a8(q[rows], s_a[rows], w, s_w)
    qd, sad, wd, swd = dev(q), dev(s_a), dev(w), dev(s_w)
    for name in ["auto", "tile_256x256", "tile_256x192", "tile_256x320", "tile_192x128"]:
        acc = torch.full((M, N), 7, dtype=torch.int32, device=DEV)
        y = prism.gemm_w8a8_variant(qd, sad, wd, swd, name, acc=acc)
        torch.cuda.synchronize()
        assert_same_ints(host(acc)[rows], acc_ref, "acc (%s)" % name)
        assert_same_floats(host(y)[rows], y_ref, "y (%s)" % name)


@pytest.mark.parametrize("M,N,K", [(600, 1300, 1056), (513, 1100, 4128), (256, 1024, 384), (1030, 2100, 2080),
                                   (300, 700, 32)])
def test_w4a8_256_row_tiles_several_column_groups(M, N, K):
    """4-bit weights on the 256-row ping-pong tiles: the packed bytes move in pairs of
    128-k stages, stages are padded to whole pairs of pairs (K = 32, 384, 1056, 2080, 4128
    leave 1-4 padded stages), and a tile's last pair already fetches the next tile's first;
    every width and the plain call give the oracle's bits on ragged shapes."""
    q, s_a, w4, s_w = _inputs(M + 5 * N + K, M, N, K, w4=True)
    y_ref, acc_ref = oracle.gemm_w4a8(q, s_a, w4, s_w)
    _run_all(prism.gemm_w4a8_variant, ["auto", "tile_256x256", "tile_256x192", "tile_256x320"], dev(q), dev(s_a),
             dev(w4), dev(s_w), y_ref, acc_ref)


@pytest.mark.parametrize("M,N,K", [(2048, 12288, 4096), (4096, 12288, 4096), (3072, 2560, 9728)])
def test_w4a8_256_row_tiles_full_size_sampled_rows(M, N, K):
    """The 4-bit shapes where the plain call picks 256-row tiles, at full size: the plain
    call and every width against the oracle on sampled rows."""
    q, s_a, w4, s_w = _inputs(M + N + K + 1, M, N, K, w4=True)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, M // 2, M - 257, M - 256, M - 1],
                                     np.random.default_rng(M + N + 1).choice(M, 16, replace=False)]))
    y_ref, acc_ref = oracle.gemm_w4a8(q[rows], s_a[rows], w4, s_w)
    qd, sad, wd, swd = dev(q), dev(s_a), dev(w4), dev(s_w)
    for name in ["auto", "tile_256x256", "tile_256x192", "tile_256x320"]:
        acc = torch.full((M, N), 7, dtype=torch.int32, device=DEV)
        y = prism.gemm_w4a8_variant(qd, sad, wd, swd, name, acc=acc)
        torch.cuda.synchronize()
        assert_same_ints(host(acc)[rows], acc_ref, "acc (%s)" % name)
        assert_same_floats(host(y)[rows], y_ref, "y (%s)" % name)


@pytest.mark.parametrize("M,N,K", [(512, 5120, 5120), (1024, 2560, 9728), (96, 17408, 2560), (128, 9728, 2560),
                                   (256, 2560, 9728), (64, 5120, 9728), (512, 2560, 2560)])
def test_few_tile_shapes_full_size_sampled_rows(M, N, K):
    """Shapes where the plain call picks 128 x 96 tiles (no split), 64 x 128
    tiles (with and without a K split) or 128 x 128 tiles with a split, at full
    size: the plain call and those entries, against the oracle on sampled rows
    (the first and last rows of 64- and 128-row tiles among them)."""
    q, s_a, w, s_w = _inputs(3 * M + N + K, M, N, K)
    fixed = [r for r in (0, 1, 63, 64, 127, 128, M // 2, M - 65, M - 64, M - 1) if 0 <= r < M]
    rows = np.unique(np.concatenate([fixed, np.random.default_rng(M * N).choice(M, min(M, 16), replace=False)]))
    y_ref, acc_ref = oracle.gemm_w8a8(q[rows], s_a[rows], w, s_w)
    qd, sad, wd, swd = dev(q), dev(s_a), dev(w), dev(s_w)
    for name in ["auto", "tile_128x96", "tile_128x96_split2", "tile_64x128", "tile_64x128_split3",
                 "tile_128x128_split3"]:
        acc = torch.full((M, N), 7, dtype=torch.int32, device=DEV)
        y = prism.gemm_w8a8_variant(qd, sad, wd, swd, name, acc=acc)
        torch.cuda.synchronize()
        assert_same_ints(host(acc)[rows], acc_ref, "acc (%s)" % name)
        assert_same_floats(host(y)[rows], y_ref, "y (%s)" % name)


def _random_shapes(seed, count):
    """Seeded (M, N, K) shapes that reach every branch of the plain call's
    dispatch: single rows, the small-M kernel (blocked and even shares), its
    boundary with the tiled path, the few-tile cost model (128 x 128,
    64 x 128, 128 x 96, K splits) and the tile-shape estimate (192, 256 and
    320 columns), with ragged M, N and K."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        M = int(rng.choice([1, 2, 5, 16, 17, 31, 32, 33, 48, 64, 65, 96, 129, 200, 257, 383, 512, 700, 1100]))
        N = int(rng.integers(1, 3200))
        K = 16 * int(rng.integers(1, 400))
        out.append((M, N, K))
    return out


@pytest.mark.parametrize("M,N,K", _random_shapes(2024, 24))
def test_plain_call_random_shapes(M, N, K):
    """The plain call on seeded random shapes: the oracle's int32 sums and
    output bits, whatever kernel, tile and split the dispatch picks."""
    q, s_a, w, s_w = _inputs(M * 7919 + N * 31 + K, M, N, K)
    y_ref, acc_ref = oracle.gemm_w8a8(q, s_a, w, s_w)
    acc = torch.full((M, N), 7, dtype=torch.int32, device=DEV)
    y = prism.gemm_w8a8(dev(q), dev(s_a), dev(w), dev(s_w), acc=acc)
    torch.cuda.synchronize()
    assert_same_ints(host(acc), acc_ref, "acc")
    assert_same_floats(host(y), y_ref, "y")


@pytest.mark.parametrize("M,N,K", [(M, N, 32 * (K // 32 + 1)) for (M, N, K) in _random_shapes(77, 12)])
def test_plain_call_random_shapes_w4a8(M, N, K):
    """The plain W4A8 call on seeded random shapes (small-M kernel with
    blocked columns or even shares, 4-bit tiled kernel with its K split)."""
    q, s_a, w4, s_w = _inputs(M * 131 + N * 7 + K, M, N, K, w4=True)
    y_ref, acc_ref = oracle.gemm_w4a8(q, s_a, w4, s_w)
    acc = torch.full((M, N), 7, dtype=torch.int32, device=DEV)
    y = prism.gemm_w4a8(dev(q), dev(s_a), dev(w4), dev(s_w), acc=acc)
    torch.cuda.synchronize()
    assert_same_ints(host(acc), acc_ref, "acc")
    assert_same_floats(host(y), y_ref, "y")


@pytest.mark.parametrize("M,N,K", [(M, N, 32 * (K // 32 + 1)) for (M, N, K) in _random_shapes(78, 12)])
def test_plain_call_random_shapes_blockscale(M, N, K):
    """The plain block-scale call on seeded random shapes (small-M block
    kernel up to 16 rows, tiled block kernel above), fp16 scales drawn as
    in the block-scale workload."""
    rng = np.random.default_rng(M * 17 + N + K)
    q = rng.integers(-128, 128, (M, K), dtype=np.int8)
    s_a = rng.uniform(1e-3, 1e-2, M).astype(np.float32)
    w = wl.int8_weights(rng, N, K)
    d = wl.block_scale_bits(rng, N, K // 32)
    y_ref, _ = oracle.gemm_w8a8_blockscale(q, s_a, w, d)
    y = prism.gemm_w8a8_blockscale(dev(q), dev(s_a), dev(w), dev(d))
    torch.cuda.synchronize()
    assert_same_floats(host(y), y_ref, "y")


@pytest.mark.parametrize("M,N,K", [(128, 2560, 9728), (100, 2052, 9728), (70, 1030, 8192), (512, 2560, 9728),
                                   (33, 5120, 5120), (300, 1000, 2048)])
def test_outputs_only_4_byte_aligned(M, N, K):
    """The C ABI asks y, acc and s_w to be 4-byte aligned only.  Called
    through the ABI directly with all three one element past a 16-byte
    boundary, the K-split launches (whose fill and epilogue kernels move 16
    bytes per access) and the other paths must still give the oracle's
    bits."""
    import ctypes
    q, s_a, w, s_w = _inputs(M + 3 * N + K, M, N, K)
    y_ref, acc_ref = oracle.gemm_w8a8(q, s_a, w, s_w)
    qd, sad, wd = dev(q), dev(s_a), dev(w)
    swb = torch.zeros(N + 1, dtype=torch.float32, device=DEV)
    swb[1:] = dev(s_w)
    yb = torch.full((M * N + 1,), 3.0, dtype=torch.float32, device=DEV)
    ab = torch.full((M * N + 1,), 7, dtype=torch.int32, device=DEV)
    P = lambda t, off=0: ctypes.c_void_p(t.data_ptr() + 4 * off)
    assert (swb.data_ptr() + 4) % 16 == 4 and (yb.data_ptr() + 4) % 16 == 4
    lib = prism.lib()
    st = ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream)
    status = lib.prism_gemm_w8a8(P(qd), P(sad), P(wd), P(swb, 1), P(yb, 1), P(ab, 1), M, N, K, st)
    torch.cuda.synchronize()
    assert status == 0
    assert_same_ints(host(ab[1:]).reshape(M, N), acc_ref, "acc")
    assert_same_floats(host(yb[1:]).reshape(M, N), y_ref, "y")
    assert host(yb[:1])[0] == 3.0 and host(ab[:1])[0] == 7   # nothing written before y / acc
