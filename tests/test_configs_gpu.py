"""GPU parity at the full sizes of the synthetic workloads (the shapes the
benchmark times), against the CPU oracle.

Where the oracle cannot do the whole workload in seconds (the block-scale
case), it checks a sample of rows: rows are independent in the definition,
so the oracle run on a subset of rows gives exactly those rows' outputs.
"""
import numpy as np
import pytest
import torch

import oracle
from exact_int8_gemm_amd import prism
from exact_int8_gemm_amd import workloads as wl
from gpu_util import DEV, assert_same_floats, assert_same_ints, dev, host

pytestmark = pytest.mark.gpu


def _quantize_both(x):
    q_ref, s_ref = oracle.quantize_rows(x)
    q, s = prism.quantize_rows(dev(x))
    torch.cuda.synchronize()
    assert_same_floats(host(s), s_ref, "scale")
    assert_same_ints(host(q), q_ref, "codes")
    return q, s, q_ref, s_ref


def test_tiny_w8a8():
    c = wl.tiny()
    q, s, q_ref, s_ref = _quantize_both(c["x"])
    y_ref, acc_ref = oracle.gemm_w8a8(q_ref, s_ref, c["w"], c["s_w"])
    acc = torch.empty(acc_ref.shape, dtype=torch.int32, device=DEV)
    y = prism.gemm_w8a8(q, s, dev(c["w"]), dev(c["s_w"]), acc=acc)
    torch.cuda.synchronize()
    assert_same_ints(host(acc), acc_ref, "acc")
    assert_same_floats(host(y), y_ref, "y")


@pytest.mark.parametrize("which", ["proj_up", "proj_down"])
def test_projection_prefill_w8a8(which):
    c = getattr(wl, which)()
    q, s, q_ref, s_ref = _quantize_both(c["x"])
    y_ref, acc_ref = oracle.gemm_w8a8(q_ref, s_ref, c["w"], c["s_w"])
    acc = torch.empty(acc_ref.shape, dtype=torch.int32, device=DEV)
    y = prism.gemm_w8a8(q, s, dev(c["w"]), dev(c["s_w"]), acc=acc)
    torch.cuda.synchronize()
    assert_same_ints(host(acc), acc_ref, "acc")
    assert_same_floats(host(y), y_ref, "y")


def test_block_scale_w8a8_sampled_rows():
    c = wl.block()
    M = c["x"].shape[0]
    q, s, q_ref, s_ref = _quantize_both(c["x"])
    y = host(prism.gemm_w8a8_blockscale(q, s, dev(c["w"]), dev(c["d"])))
    rows = np.unique(np.concatenate([[0, 1, 127, 128, M - 1], np.random.default_rng(11).choice(M, 43, replace=False)]))
    y_ref, _ = oracle.gemm_w8a8_blockscale(q_ref[rows], s_ref[rows], c["w"], c["d"])
    assert_same_floats(y[rows], y_ref, "y sampled rows")


@pytest.mark.parametrize("M", [1, 4, 16, 64])
def test_w4a8_decode(M):
    c = wl.w4()
    x = c["x"][:M]
    q, s, q_ref, s_ref = _quantize_both(x)
    y_ref, acc_ref = oracle.gemm_w4a8(q_ref, s_ref, c["w4"], c["s_w"])
    acc = torch.empty(acc_ref.shape, dtype=torch.int32, device=DEV)
    y = prism.gemm_w4a8(q, s, dev(c["w4"]), dev(c["s_w"]), acc=acc)
    torch.cuda.synchronize()
    assert_same_ints(host(acc), acc_ref, "acc")
    assert_same_floats(host(y), y_ref, "y")


def test_batch_invariance_stress():
    """64 probe rows alone (M = 1 each), overwriting rows of an 8192-row batch,
    and inserted into it (8256 rows): every probe row must be bit-identical
    across the three runs, across repeats, and equal to the oracle."""
    st = wl.stress()
    w, s_w = dev(st["w"]), dev(st["s_w"])
    probes = st["x_probe"]
    q_ref, s_ref = oracle.quantize_rows(probes)
    y_ref, _ = oracle.gemm_w8a8(q_ref, s_ref, st["w"], st["s_w"])

    def run(x):
        q, s = prism.quantize_rows(dev(x))
        return host(prism.gemm_w8a8(q, s, w, s_w))

    alone = np.concatenate([run(probes[j:j + 1]) for j in range(probes.shape[0])])
    assert_same_floats(alone, y_ref, "probes alone vs oracle")
    x_over, where_over = wl.stress_overwrite(st)
    x_ins, where_ins = wl.stress_insert(st)
    assert x_ins.shape[0] == 8256
    for rep in range(2):
        y_over = run(x_over)
        assert_same_floats(y_over[where_over], alone, "overwrite reading, repeat %d" % rep)
        y_ins = run(x_ins)
        assert_same_floats(y_ins[where_ins], alone, "insert reading, repeat %d" % rep)
