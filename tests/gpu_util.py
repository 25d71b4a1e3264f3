"""Helpers for the GPU parity tests: device transfer and bitwise comparison.

Inputs come from ``exact_int8_gemm_amd.workloads`` (seeded numpy), the
expected values from the CPU oracle; the GPU side runs through the C ABI via
``exact_int8_gemm_amd.prism``.  Floats are compared as bit patterns (so -0.0
and +0.0 differ); two NaNs count as equal, whatever their payloads.
"""
import numpy as np
import torch

DEV = torch.device("cuda:0")


def dev(a):
    a = np.ascontiguousarray(a)
    if not a.flags.writeable:
        a = a.copy()
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(DEV)


def host(t):
    return t.detach().cpu().numpy()


def assert_same_floats(got, exp, what=""):
    got = np.ascontiguousarray(got, np.float32)
    exp = np.ascontiguousarray(exp, np.float32)
    assert got.shape == exp.shape, (what, got.shape, exp.shape)
    gn, en = np.isnan(got), np.isnan(exp)
    same = (got.view(np.uint32) == exp.view(np.uint32)) | (gn & en)
    if not same.all():
        idx = np.argwhere(~same)
        first = tuple(int(v) for v in idx[0])
        raise AssertionError("%s: %d of %d floats differ; first at %s: got %r (0x%08x) expected %r (0x%08x)" % (
            what, len(idx), got.size, first, float(got[first]), int(got.view(np.uint32)[first]),
            float(exp[first]), int(exp.view(np.uint32)[first])))


def assert_same_ints(got, exp, what=""):
    got, exp = np.asarray(got), np.asarray(exp)
    assert got.shape == exp.shape, (what, got.shape, exp.shape)
    if not np.array_equal(got, exp):
        idx = np.argwhere(got != exp)
        first = tuple(int(v) for v in idx[0])
        raise AssertionError("%s: %d of %d ints differ; first at %s: got %d expected %d" % (
            what, len(idx), got.size, first, int(got[first]), int(exp[first])))
