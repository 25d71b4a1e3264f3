"""GPU: the measurement kernels compute what they claim, so that the rates bench.py
derives from them count real work.

* prism_peak_read: the XOR of its parts equals the XOR of every 32-bit word of the
  buffer (every byte read once, none dropped), on sizes from one 16-byte piece to a
  buffer larger than one pass of the grid.
* prism_peak_fold: the int8 and f16 MFMA forms of the block fold write the same bits
  (each 32-k block sum is exact either way), and so do the two MFMA-only forms.
* prism_peak_mfma: each thread's checksum equals a CPU model of the MFMA loop.  The
  model needs only the row/column roles of the 32x32x32 int8 MFMA (lane l holds row
  l % 32 of A and column l % 32 of B for one half of k, lanes l and l + 32 the two
  halves; output register r of lane l is C[8 (r / 4) + 4 (l / 32) + r % 4][l % 32]) and
  that A and B place their k in the same bytes of a lane: C = A_0 B_0^T + A_1 B_1^T
  over the lanes' 16 bytes, whatever k each byte stands for.
"""
import numpy as np
import pytest
import torch

from exact_int8_gemm_amd import prism
from gpu_util import DEV

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, 1 << 20, 25 * (1 << 20) + 48, 600 << 20])
def test_peak_read_reads_every_word_once(nbytes):
    rng = np.random.default_rng(nbytes % 1000)
    host = rng.integers(0, 2 ** 32, nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to(DEV)
    parts = prism.peak_read(buf)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(parts.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)


def _fragments(salt, seed):
    """[64 lanes, 16 bytes] int8: the top byte of (37 l + 101 j + 7919 salt + 13 seed) * 2654435761."""
    lane = np.arange(64, dtype=np.uint64)[:, None]
    j = np.arange(16, dtype=np.uint64)[None, :]
    h = ((37 * lane + 101 * j + 7919 * salt + 13 * seed) * 2654435761) % 2 ** 32
    return (h >> 24).astype(np.uint8).view(np.int8).astype(np.int64)


def _mfma_model(iters, wps, seed):
    C = np.zeros((32, 32), np.int64)
    for sa, sb in ((0, 1), (2, 3)):   # one step with (A0, B0), one with (A1, B1)
        A, B = _fragments(sa, seed), _fragments(sb, seed)
        C += A[:32] @ B[:32].T + A[32:] @ B[32:].T
    nacc = 8 if wps < 4 else 4
    C *= iters * (16 // nacc) // 2
    lane = np.arange(64)
    s = np.zeros(64, np.int64)
    for r in range(16):
        rows = 8 * (r // 4) + 4 * (lane // 32) + r % 4
        s += C[rows, lane % 32]
    return (nacc * s) % 2 ** 32


@pytest.mark.parametrize("wps", [1, 2, 4])
@pytest.mark.parametrize("iters,seed", [(1, 0), (3, 12345), (50, 7)])
def test_peak_mfma_checksums(wps, iters, seed):
    out = prism.peak_mfma(iters, wps, seed)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32).astype(np.int64)
    want = _mfma_model(iters, wps, seed)
    threads = 128 * wps
    assert got.size % threads == 0
    got = got.reshape(-1, threads)
    for t in range(threads):
        assert (got[:, t] == want[t % 64]).all(), (t, got[:, t][:4], want[t % 64])


@pytest.mark.parametrize("iters", [1, 2, 7, 32])
def test_peak_fold_int8_and_f16_forms_agree(iters):
    a = prism.peak_fold(0, iters)
    b = prism.peak_fold(1, iters)
    c = prism.peak_fold(2, iters)
    d = prism.peak_fold(3, iters)
    e = prism.peak_fold(4, iters)
    torch.cuda.synchronize()
    a, b, c, d, e = (t.cpu().numpy() for t in (a, b, c, d, e))
    assert np.isfinite(a).all() and np.isfinite(e).all()
    assert (a != 0).any() and (c != 0).any()
    assert np.array_equal(a.view(np.int32), b.view(np.int32))
    assert np.array_equal(c.view(np.int32), d.view(np.int32))
