"""Batch invariance on the GPU: a row's outputs do not depend on the batch
size, on its position in the batch (first, middle, last, ragged tail of a
tile), on which kernel family the row count selects, on repetition, or on
concurrent work in another stream.  Compared bit for bit.
"""
import numpy as np
import pytest
import torch

from exact_int8_gemm_amd import prism
from exact_int8_gemm_amd import workloads as wl
from gpu_util import DEV, assert_same_floats, dev, host

pytestmark = pytest.mark.gpu

BATCHES = [1, 2, 16, 17, 64, 65, 128, 255, 256, 257, 1000, 4096]


def _rows(seed, M, K):
    return np.random.default_rng(seed).standard_normal((M, K), dtype=np.float32)


def _gemm(kind, x, c):
    q, s = prism.quantize_rows(dev(x))
    if kind == "w8a8":
        return host(prism.gemm_w8a8(q, s, c["w_d"], c["s_w_d"]))
    if kind == "w4a8":
        return host(prism.gemm_w4a8(q, s, c["w4_d"], c["s_w_d"]))
    return host(prism.gemm_w8a8_blockscale(q, s, c["w_d"], c["d_d"]))


@pytest.fixture(scope="module", params=["w8a8", "w4a8", "block"])
def setup(request):
    kind = request.param
    N, K = 520, 1056
    c = wl.random_case(5, 1, N, K, "w4a8" if kind == "w4a8" else ("block" if kind == "block" else "w8a8"))
    out = {"kind": kind}
    if "w" in c:
        out["w_d"] = dev(c["w"])
    if "w4" in c:
        out["w4_d"] = dev(c["w4"])
    if "s_w" in c:
        out["s_w_d"] = dev(c["s_w"])
    if "d" in c:
        out["d_d"] = dev(c["d"])
    out["K"] = K
    probe = _rows(77, 1, K)
    out["probe"] = probe
    out["alone"] = _gemm(kind, probe, out)
    return out


@pytest.mark.parametrize("M", BATCHES)
def test_row_position_and_batch_size(setup, M):
    K = setup["K"]
    x = _rows(1000 + M, M, K)
    for p in sorted({0, M // 2, M - 1}):
        xb = x.copy()
        xb[p] = setup["probe"][0]
        y = _gemm(setup["kind"], xb, setup)
        assert_same_floats(y[p:p + 1], setup["alone"], "%s M=%d position %d" % (setup["kind"], M, p))


def test_repeat_runs_identical(setup):
    x = _rows(5, 300, setup["K"])
    first = _gemm(setup["kind"], x, setup)
    for _ in range(9):
        assert_same_floats(_gemm(setup["kind"], x, setup), first, "repeat")


def test_concurrent_streams_identical(setup):
    x = _rows(6, 700, setup["K"])
    ref = _gemm(setup["kind"], x, setup)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    xd = dev(x)
    torch.cuda.synchronize()
    outs = []
    for st in (s1, s2, s1, s2):
        with torch.cuda.stream(st):
            q, s = prism.quantize_rows(xd)
            if setup["kind"] == "w8a8":
                outs.append(prism.gemm_w8a8(q, s, setup["w_d"], setup["s_w_d"]))
            elif setup["kind"] == "w4a8":
                outs.append(prism.gemm_w4a8(q, s, setup["w4_d"], setup["s_w_d"]))
            else:
                outs.append(prism.gemm_w8a8_blockscale(q, s, setup["w_d"], setup["d_d"]))
    torch.cuda.synchronize()
    for o in outs:
        assert_same_floats(host(o), ref, "stream")
