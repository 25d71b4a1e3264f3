"""Seeded random shapes through the whole path (GPU): quantize, then the GEMM
of each weight format, compared bit for bit with the CPU oracle.

The fixed tests pin chosen tile boundaries; these cases draw M, N and K at
random (M log-uniform up to 1200, K a multiple of the format's granule) so that
ragged tails land in places no one picked.  Every case is printed in its test
id, and the draw is a pure function of the case number.
"""
import numpy as np
import pytest
import torch

import oracle
from exact_int8_gemm_amd import prism
from exact_int8_gemm_amd import workloads as wl
from gpu_util import DEV, assert_same_floats, assert_same_ints, dev, host

pytestmark = pytest.mark.gpu

KINDS = ["w8a8", "w4a8", "block", "q4k"]


def _draw(i):
    r = np.random.default_rng(90210 + i)
    kind = KINDS[i % 4]
    M = int(np.exp(r.uniform(0, np.log(1200))))
    if kind == "q4k":
        N, K = int(r.integers(1, 200)), 256 * int(r.integers(1, 5))
    else:
        g = 16 if kind == "w8a8" else 32
        N, K = int(r.integers(1, 2500)), g * int(r.integers(1, 6000 // g))
    while M * N * K > 2e9:   # keep the oracle to a fraction of a second
        M = max(1, M // 2)
    return kind, M, N, K


def _draw_wide(i):
    """More than 16384 columns and at most 160 rows, where the plain calls
    choose between the small-M kernel and 64-row tiles by M."""
    r = np.random.default_rng(31337 + i)
    kind = "w8a8" if i % 2 == 0 else "w4a8"
    M = int(np.exp(r.uniform(0, np.log(160))))
    g = 16 if kind == "w8a8" else 32
    N, K = int(r.integers(16385, 40000)), g * int(r.integers(1, 2048 // g))
    while M * N * K > 2e9:
        M = max(1, M // 2)
    return kind, M, N, K


CASES = [_draw(i) for i in range(48)] + [_draw_wide(i) for i in range(16)]


@pytest.mark.parametrize("kind,M,N,K", CASES, ids=["%s-M%d-N%d-K%d" % c for c in CASES])
def test_random_shape(kind, M, N, K):
    rng = np.random.default_rng(M * 131 + N * 17 + K)
    x = wl.activations(rng, M, K)
    q_ref, s_ref = oracle.quantize_rows(x)
    q, s = prism.quantize_rows(dev(x))
    assert_same_ints(host(q), q_ref, "q")
    assert_same_floats(host(s), s_ref, "s_a")
    if kind == "q4k":
        from test_oracle_pins import _pack_q4_k, _q4k_case
        blocks = _pack_q4_k(*_q4k_case(M + N + K, N, K))
        w4, hdr = prism.repack_q4_k(dev(blocks), N, K)
        y = prism.gemm_w4a8_q4k(q, s, w4, hdr)
        torch.cuda.synchronize()
        assert_same_floats(host(y), oracle.gemm_w4a8_q4k(q_ref, s_ref, blocks, N), "y")
        return
    c = wl.random_case(M + N + K, 1, N, K, kind)
    if kind == "block":
        y_ref, _ = oracle.gemm_w8a8_blockscale(q_ref, s_ref, c["w"], c["d"])
        y = prism.gemm_w8a8_blockscale(q, s, dev(c["w"]), dev(c["d"]))
        torch.cuda.synchronize()
        assert_same_floats(host(y), y_ref, "y")
        return
    acc = torch.empty((M, N), dtype=torch.int32, device=DEV)
    if kind == "w4a8":
        y_ref, acc_ref = oracle.gemm_w4a8(q_ref, s_ref, c["w4"], c["s_w"])
        y = prism.gemm_w4a8(q, s, dev(c["w4"]), dev(c["s_w"]), acc=acc)
    else:
        y_ref, acc_ref = oracle.gemm_w8a8(q_ref, s_ref, c["w"], c["s_w"])
        y = prism.gemm_w8a8(q, s, dev(c["w"]), dev(c["s_w"]), acc=acc)
    torch.cuda.synchronize()
    assert_same_ints(host(acc), acc_ref, "acc")
    assert_same_floats(host(y), y_ref, "y")
