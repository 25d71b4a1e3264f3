"""HIP graph capture of the library's calls (GPU).

Every entry point launches kernels only (no allocation, no memset: a K-split
launch clears y with a fill kernel), so a captured sequence can be replayed.
Each replay must give the bits of the eager calls, also with other work and
synchronisation between the replays.
"""
import numpy as np
import pytest
import torch

import oracle
from exact_int8_gemm_amd import prism
from exact_int8_gemm_amd import workloads as wl
from gpu_util import DEV, assert_same_floats, dev, host

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    rng = np.random.default_rng(2024)
    M, K1, N1 = 100, 9728, 2560     # few tiles, long K: the K-split path (fill, atomics, finalize)
    M2, K2, N2 = 8, 1024, 700       # small-M path, 4-bit weights
    x1 = dev(rng.standard_normal((M, K1), dtype=np.float32))
    w1, s1 = dev(wl.int8_weights(rng, N1, K1)), dev(wl.channel_scales(rng, N1))
    x2 = dev(rng.standard_normal((M2, K2), dtype=np.float32))
    w4 = dev(wl.pack_int4(rng.integers(-8, 8, (N2, K2), dtype=np.int8)))
    s2 = dev(wl.channel_scales(rng, N2))
    wb = dev(wl.int8_weights(rng, 300, K2))
    db = dev(wl.block_scale_bits(rng, 300, K2 // 32))

    q1 = torch.empty((M, K1), dtype=torch.int8, device=DEV)
    a1 = torch.empty((M,), dtype=torch.float32, device=DEV)
    y1 = torch.empty((M, N1), dtype=torch.float32, device=DEV)
    q2 = torch.empty((M2, K2), dtype=torch.int8, device=DEV)
    a2 = torch.empty((M2,), dtype=torch.float32, device=DEV)
    y2 = torch.empty((M2, N2), dtype=torch.float32, device=DEV)
    y3 = torch.empty((M2, 300), dtype=torch.float32, device=DEV)

    def calls():
        prism.quantize_rows(x1, q=q1, scale=a1)
        prism.gemm_w8a8(q1, a1, w1, s1, y=y1)
        prism.quantize_rows_static(x2, 0.05, q=q2, scale=a2)
        prism.gemm_w4a8(q2, a2, w4, s2, y=y2)
        prism.gemm_w8a8_blockscale(q2, a2, wb, db, y=y3)

    # eager reference (also the warm-up the capture needs), checked against the oracle
    side = torch.cuda.Stream(device=DEV)
    side.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream(DEV).wait_stream(side)
    torch.cuda.synchronize()
    ref = [host(t).copy() for t in (y1, y2, y3)]
    qr, sr = oracle.quantize_rows(host(x1))
    assert_same_floats(ref[0], oracle.gemm_w8a8(qr, sr, host(w1), host(s1))[0], "eager y1")

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    for rep in range(4):
        for t in (y1, y2, y3):
            t.fill_(float("nan"))        # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, exp, name in zip((y1, y2, y3), ref, ("w8a8 split-K", "w4a8 small-M", "block-scale")):
            assert_same_floats(host(got), exp, "%s, replay %d" % (name, rep))
