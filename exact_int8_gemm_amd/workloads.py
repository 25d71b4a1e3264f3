"""Seeded synthetic inputs for the exact int8 linear layer.

This module draws random numbers and packs them into the input formats; it
holds none of the layer's arithmetic (no quantization, no sums, no scaling),
so that the GPU path and the CPU oracle can both take their inputs from it.

The pages publish no weights and no evaluation data: StartLux-Prism measures
on released model files and on evaluation suites ("Performance" and
"Accuracy" sections of its README), none of which is available here.  These
generators stand in for them with the shapes and value distributions of an
int8 (Q8_0-style) or 4-bit model's projections:

* ``tiny``        M=8, K=512, N=256 (seed 0)
* ``proj_up``     M=512, K=2560, N=9728, 1% outlier activation columns x20 (seed 1)
* ``proj_down``   M=512, K=9728, N=2560, same recipe (seed 2)
* ``block``       M=2048, K=5120, N=17408, fp16 block scales |N(0,0.02)|/127 (seed 3)
* ``w4``          K=4096, N=12288, int4 in [-8,7] packed low nibble first,
                  64 activation rows of which the first M in {1,4,16,64} are used (seed 4)
* ``stress``      K=N=5120; 64 probe rows (seed 6) placed at random positions
                  (seed 8) among 8192 background rows (seed 7); weights seed 5

Weights are uniform integers in [-127, 127]; per-channel scales are uniform
in [1e-3, 1e-2] (fp32); activations are fp32 N(0, 1).  Draws happen in the
order written below, from ``numpy.random.default_rng(seed)`` (PCG64).
"""
from __future__ import annotations

import numpy as np


def int8_weights(rng, n, k):
    return rng.integers(-127, 128, size=(n, k), dtype=np.int8)


def channel_scales(rng, n):
    return rng.uniform(1e-3, 1e-2, size=n).astype(np.float32)


def activations(rng, m, k):
    return rng.standard_normal((m, k), dtype=np.float32)


def pack_int4(w):
    """Signed values in [-8, 7], [N, K] -> bytes [N, K/2]; byte j holds k=2j in
    its low nibble and k=2j+1 in its high nibble, both two's complement."""
    w = np.asarray(w, dtype=np.int16)
    if w.ndim != 2 or w.shape[1] % 2:
        raise ValueError("need [N, K] with K even")
    if w.min(initial=0) < -8 or w.max(initial=0) > 7:
        raise ValueError("int4 values must lie in [-8, 7]")
    lo = (w[:, 0::2] & 15).astype(np.uint8)
    hi = (w[:, 1::2] & 15).astype(np.uint8)
    return (lo | (hi << 4)).astype(np.uint8)


def tiny():
    rng = np.random.default_rng(0)
    w = int8_weights(rng, 256, 512)
    s_w = channel_scales(rng, 256)
    x = activations(rng, 8, 512)
    return dict(x=x, w=w, s_w=s_w)


def _projection(seed, m, k, n):
    rng = np.random.default_rng(seed)
    w = int8_weights(rng, n, k)
    s_w = channel_scales(rng, n)
    x = activations(rng, m, k)
    cols = rng.choice(k, size=int(round(0.01 * k)), replace=False)
    x[:, cols] *= np.float32(20.0)
    return dict(x=x, w=w, s_w=s_w, outlier_cols=np.sort(cols))


def proj_up(m=512):
    """4B-class MLP up-projection: K=2560, N=9728."""
    return _projection(1, m, 2560, 9728)


def proj_down(m=512):
    """4B-class MLP down-projection: K=9728, N=2560."""
    return _projection(2, m, 9728, 2560)


def block_scale_bits(rng, n, nblocks):
    """fp16 scales |N(0, 0.02)| / 127, rounded to binary16 (RNE), as uint16 bit patterns."""
    d = np.abs(rng.normal(0.0, 0.02, size=(n, nblocks))) / 127.0
    return d.astype(np.float16).view(np.uint16)


def block(m=2048, k=5120, n=17408):
    rng = np.random.default_rng(3)
    w = int8_weights(rng, n, k)
    d = block_scale_bits(rng, n, k // 32)
    x = activations(rng, m, k)
    return dict(x=x, w=w, d=d)


def w4(k=4096, n=12288, rows=64):
    rng = np.random.default_rng(4)
    wv = rng.integers(-8, 8, size=(n, k), dtype=np.int8)
    s_w = channel_scales(rng, n)
    x = activations(rng, rows, k)
    return dict(x=x, w4=pack_int4(wv), s_w=s_w)


def stress(background=8192, probes=64, k=5120, n=5120):
    w_rng = np.random.default_rng(5)
    w = int8_weights(w_rng, n, k)
    s_w = channel_scales(w_rng, n)
    x_probe = activations(np.random.default_rng(6), probes, k)
    x_bg = activations(np.random.default_rng(7), background, k)
    pos = np.random.default_rng(8).choice(background, size=probes, replace=False)
    return dict(w=w, s_w=s_w, x_probe=x_probe, x_bg=x_bg, pos=pos)


def stress_overwrite(st):
    """Reading (i): M = background rows, probe j overwrites row pos[j]."""
    x = st["x_bg"].copy()
    x[st["pos"]] = st["x_probe"]
    return x, st["pos"]


def stress_insert(st):
    """Reading (ii): M = background + probes, probe j inserted before background row pos[j]."""
    bg, pr, pos = st["x_bg"], st["x_probe"], st["pos"]
    order = np.argsort(pos, kind="stable")
    out, where, prev = [], np.empty(len(pos), np.int64), 0
    row = 0
    for j in order:
        p = int(pos[j])
        out.append(bg[prev:p])
        row += p - prev
        out.append(pr[j:j + 1])
        where[j] = row
        row += 1
        prev = p
    out.append(bg[prev:])
    return np.concatenate(out, axis=0), where


def random_case(seed, m, n, k, kind="w8a8"):
    """Small seeded case of any shape, for sweeps over tiles and ragged tails."""
    rng = np.random.default_rng(seed)
    x = activations(rng, m, k)
    if kind == "w4a8":
        wv = rng.integers(-8, 8, size=(n, k), dtype=np.int8)
        return dict(x=x, w4=pack_int4(wv), s_w=channel_scales(rng, n))
    w = int8_weights(rng, n, k)
    if kind == "block":
        return dict(x=x, w=w, d=block_scale_bits(rng, n, k // 32))
    return dict(x=x, w=w, s_w=channel_scales(rng, n))
