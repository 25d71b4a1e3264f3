#!/usr/bin/env python3
"""Benchmark of the exact int8 linear layer on one MI355X.

A step is one pass of the hot path over the largest single-GPU workload, the
batch-invariance stress batch (W8A8 with per-channel scales):
    quantize rows of X [8192 x 5120]  -> GEMM with W [5120 x 5120]
(X holds the 64 seeded probe rows at seeded positions among N(0,1) rows).
Inputs are synthetic and seeded (exact_int8_gemm_amd.workloads) and resident
in HBM before timing starts.  R copies of every input set are rotated so that
the working set exceeds the 256 MB MALL plus L2, so operands come from HBM.

Printed: one JSON line with the whole-step int8 throughput (TOPS), the
roofline of the GEMM (measured with HIP events around its launches, in a
second pass of the same steps right after the timed one: the timed steps
carry no events), the CPU oracle's throughput on a bounded sample, and
per-kernel measurements of the other workloads (the M = 512 projection step,
W4A8 decode and prefill, block-scale, Q4_K, repacks, decode) under "kernels".
Those measurements run after the headline's inputs are on the GPU and before
its warm-up steps, so the warm-up and timed steps start on a GPU at its steady
clocks.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5000.0      # MI355X dense int8 MFMA, 5.0 POP/s
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, 8 TB/s
METRIC = "int8 TOPS (and GB/s at small M) as % of MI355X roofline, bit-exact"
ROTATE_BYTES = 640 << 20     # rotate input copies until the working set exceeds this


def _args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-kernels", action="store_true", help="skip the per-kernel measurements of other workloads")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 256 MiB device copy three times (scale for HBM byte counters)")
    ap.add_argument("--only", default=None, help="run only one kernel measurement (for profiling): "
                    "step | proj | w4a8 | block | repack | q4k | decode | vendor | stress | peaks | sweep (M sweep, not in the default run)")
    return ap.parse_args()


class Launcher:
    """Direct ctypes calls of the C ABI with pointers resolved once (no per-call checks)."""

    def __init__(self, prism, stream):
        self.lib = prism.lib()
        self.stream = ctypes.c_void_p(stream)

    @staticmethod
    def p(t):
        return ctypes.c_void_p(t.data_ptr())

    def quantize(self, x, q, s):
        M, K = x.shape
        f, a = self.lib.prism_quantize_rows, (self.p(x), self.p(q), self.p(s), M, K, self.stream)
        return lambda: f(*a)

    def quantize_static(self, x, q, s, scale):
        M, K = x.shape
        f, a = self.lib.prism_quantize_rows_static, (self.p(x), self.p(q), self.p(s), ctypes.c_float(scale), M, K,
                                                     self.stream)
        return lambda: f(*a)

    def repack(self, blocks, w, d):
        N, K = w.shape
        f, a = self.lib.prism_repack_q8_0, (self.p(blocks), self.p(w), self.p(d), N, K, self.stream)
        return lambda: f(*a)

    def repack_q4k(self, blocks, w4, hdr):
        N, K = w4.shape[0], 2 * w4.shape[1]
        f, a = self.lib.prism_repack_q4_k, (self.p(blocks), self.p(w4), self.p(hdr), N, K, self.stream)
        return lambda: f(*a)

    def q4k(self, q, sa, w4, hdr, y):
        M, K = q.shape
        N = w4.shape[0]
        f, a = self.lib.prism_gemm_w4a8_q4k, (self.p(q), self.p(sa), self.p(w4), self.p(hdr), self.p(y),
                                              M, N, K, self.stream)
        return lambda: f(*a)

    def w8a8(self, q, sa, w, sw, y):
        M, K = q.shape
        N = w.shape[0]
        f, a = self.lib.prism_gemm_w8a8, (self.p(q), self.p(sa), self.p(w), self.p(sw), self.p(y), None, M, N, K,
                                          self.stream)
        return lambda: f(*a)

    def quantize_w8a8(self, x, q, sa, w, sw, y):
        M, K = x.shape
        N = w.shape[0]
        f, a = self.lib.prism_quantize_gemm_w8a8, (self.p(x), self.p(q), self.p(sa), self.p(w), self.p(sw), self.p(y),
                                                   None, M, N, K, self.stream)
        return lambda: f(*a)

    def w4a8(self, q, sa, w4, sw, y):
        M, K = q.shape
        N = w4.shape[0]
        f, a = self.lib.prism_gemm_w4a8, (self.p(q), self.p(sa), self.p(w4), self.p(sw), self.p(y), None, M, N, K,
                                          self.stream)
        return lambda: f(*a)

    def block(self, q, sa, w, d, y):
        M, K = q.shape
        N = w.shape[0]
        f, a = self.lib.prism_gemm_w8a8_blockscale, (self.p(q), self.p(sa), self.p(w), self.p(d), self.p(y), None,
                                                     M, N, K, self.stream)
        return lambda: f(*a)


def _check(status):
    if status != 0:
        raise RuntimeError("prism call failed with status %d" % status)


def _copies(bytes_per_set):
    return max(2, -(-ROTATE_BYTES // max(1, bytes_per_set)))


# Sources of the per-channel W8A8 GEMM path of M > 64 (dispatch, tiled and
# persistent kernels, direct-to-LDS copies): a traffic figure is used only if
# it was measured on exactly these sources.
KERNEL_SOURCES = ["gemm_tiled_kernels.h", "gemm_pingpong.h", "gemm_tiled.hip", "lds_copy.h", "prism_abi.cpp",
                  "prism_internal.h"]


def _src_hash(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "exact_int8_gemm_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic(kernel_key, src_hash):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic_" + kernel_key + ".md")
    if not os.path.exists(path):
        return None
    for line in open(path):
        line = line.strip()
        if line.startswith("{") and '"traffic_bytes"' in line:
            rec = json.loads(line)
            if rec.get("src_hash") == src_hash:
                return rec["traffic_bytes"]
    return None


# --------------------------------------------------------------------- steps

def _gemm_roofline(name, M, N, K, us, traffic_key, src):
    """Roofline record of one W8A8 per-channel GEMM launch taking `us` microseconds."""
    ops = 2 * M * N * K
    nbytes = N * K + 4 * N + M * K + 4 * M + 4 * M * N  # W, s_w, q, s_a, y
    t = us / 1e6
    if ops / (PEAK_INT8_TOPS * 1e12) >= nbytes / (PEAK_HBM_GBS * 1e9):
        rec = dict(bound="mfma", achieved=ops / t / 1e12, peak=PEAK_INT8_TOPS, unit="TOPS")
    else:
        rec = dict(bound="hbm", achieved=nbytes / t / 1e9, peak=PEAK_HBM_GBS, unit="GB/s")
    rec["frac"] = rec["achieved"] / rec["peak"]
    rec["traffic"] = _traffic(traffic_key, src)
    rec.update(launch="%s, prism_gemm_w8a8 (M=%d, K=%d, N=%d)" % (name, M, K, N), avg_launch_us=us,
               ops_per_launch=ops, algorithmic_bytes_per_launch=nbytes, mfma_frac=ops / t / 1e12 / PEAK_INT8_TOPS,
               hbm_frac=nbytes / t / 1e9 / PEAK_HBM_GBS)
    return rec


def run_steps(torch, prism, cases, steps, warmup):
    """Times `steps` steps; a step runs, for each case (x, w, s_w), the row quantizer
    on x and then the W8A8 GEMM of its codes with w.  R copies of every case's
    buffers are rotated so that the working set exceeds the MALL and L2.

    The timed steps carry no events (a timing event between two kernels costs a
    few microseconds of its own on this GPU); the per-launch durations come from
    a second pass of the same steps with HIP events recorded on the launch
    stream around each quantizer and each GEMM call."""
    return prepare_steps(torch, prism, cases)(steps, warmup)


def prepare_steps(torch, prism, cases):
    """The buffers and launchers of run_steps (inputs copied to the GPU); returns
    the function that runs the warm-up, timed and event passes."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    L = Launcher(prism, stream.cuda_stream)

    def T(a):
        return torch.from_numpy(a).to(dev)

    per_set = sum(c["x"].nbytes + c["w"].nbytes + c["x"].shape[0] * (c["x"].shape[1] + 4 + 4 * c["w"].shape[0])
                  for c in cases)
    R = _copies(per_set)
    sets = []
    for _ in range(R):
        s = []
        for c in cases:
            Mx, K = c["x"].shape
            N = c["w"].shape[0]
            x, w, sw = T(c["x"]), T(c["w"]), T(c["s_w"])
            q = torch.empty((Mx, K), dtype=torch.int8, device=dev)
            sa = torch.empty((Mx,), dtype=torch.float32, device=dev)
            y = torch.empty((Mx, N), dtype=torch.float32, device=dev)
            # the launchers hold raw pointers only: keep every tensor referenced here
            s.append(dict(quant=L.quantize(x, q, sa), gemm=L.w8a8(q, sa, w, sw, y), x=x, w=w, sw=sw, y=y, q=q,
                          sa=sa))
        sets.append(s)
    torch.cuda.synchronize()
    nc = len(cases)

    def step(i, record):
        for j, p in enumerate(sets[i % R]):
            if record is not None:
                record[j][0].record(stream)
            _check(p["quant"]())
            if record is not None:
                record[j][1].record(stream)
            _check(p["gemm"]())
            if record is not None:
                record[j][2].record(stream)

    def run(steps, warmup):
        E = torch.cuda.Event
        ev = [[[E(enable_timing=True) for _ in range(3)] for _ in range(nc)] for _ in range(steps)]
        for i in range(warmup):
            step(i, None)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            step(i, None)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        for i in range(steps):
            step(i, ev[i])
        torch.cuda.synchronize()
        quant_us = [sum(ev[i][j][0].elapsed_time(ev[i][j][1]) for i in range(steps)) / steps * 1e3 for j in range(nc)]
        gemm_us = [sum(ev[i][j][1].elapsed_time(ev[i][j][2]) for i in range(steps)) / steps * 1e3 for j in range(nc)]
        last = sets[(steps - 1) % R]
        return dict(ms_per_step=wall * 1e3 / steps, R=R, quant_us=quant_us, gemm_us=gemm_us,
                    outputs=[(p["q"], p["sa"], p["y"]) for p in last])

    return run


def headline(torch, prism, wl, args, before_timing=None):
    """The largest single-GPU workload: the batch-invariance stress batch (M = 8192
    rows of K = 5120, the 64 probe rows placed among them) quantized per row and
    multiplied with the 5120 x 5120 int8 weights (per-channel scales).
    before_timing runs after the inputs are on the GPU and before the warm-up
    steps (the default run puts the per-kernel measurements there)."""
    st = wl.stress()
    x, _ = wl.stress_overwrite(st)
    case = dict(x=x, w=st["w"], s_w=st["s_w"])
    M, K = x.shape
    N = st["w"].shape[0]
    run = prepare_steps(torch, prism, [case])
    extra = before_timing() if before_timing is not None else None
    r = run(args.steps, args.warmup)
    src = _src_hash(KERNEL_SOURCES)
    roof = _gemm_roofline("stress GEMM", M, N, K, r["gemm_us"][0], "gemm_w8a8_stress_m8192", src)
    roof["timing"] = "HIP events on the launch stream around each GEMM call, over a second pass of the timed steps"
    qus = r["quant_us"][0]
    qbytes = 5 * M * K + 4 * M
    roof["quantizer"] = dict(launch="prism_quantize_rows (M=%d, K=%d)" % (M, K), avg_launch_us=qus,
                             bound="hbm", achieved=qbytes / qus / 1e3, peak=PEAK_HBM_GBS, unit="GB/s",
                             frac=qbytes / qus / 1e3 / PEAK_HBM_GBS, algorithmic_bytes_per_launch=qbytes)
    ops = 2 * M * N * K
    return dict(value=ops / (r["ms_per_step"] / 1e3) / 1e12, ms_per_step=r["ms_per_step"], R=r["R"], M=M, N=N, K=K,
                roofline=roof, outputs=r["outputs"], case=case, extra=extra)


def proj_step(torch, prism, wl, steps=100, warmup=10):
    """The 4B-class projection prefill step (M = 512): quantize + GEMM for the
    up-projection (K = 2560, N = 9728) and the down-projection (K = 9728, N = 2560)."""
    up, dn = wl.proj_up(), wl.proj_down()
    M = up["x"].shape[0]
    r = run_steps(torch, prism, [up, dn], steps, warmup)
    src = _src_hash(KERNEL_SOURCES)
    gemms = [_gemm_roofline("%s GEMM" % name, M, c["w"].shape[0], c["x"].shape[1], r["gemm_us"][j], "gemm_w8a8_" + key,
                            src)
             for j, (c, name, key) in enumerate(((up, "up-projection", "proj_up"), (dn, "down-projection",
                                                                                     "proj_down")))]
    ops = 2 * (2 * M * 2560 * 9728)
    return dict(tops=ops / (r["ms_per_step"] / 1e3) / 1e12, ms_per_step=r["ms_per_step"], us=r["ms_per_step"] * 1e3,
                quantize_us=r["quant_us"], copies=r["R"], gemms=gemms)


# --------------------------------------------------------------- other kernels

def _time_launches(torch, fns, reps):
    """(single, stream): average duration (s) of launches cycled from fns when each
    is bracketed by its own pair of events, and when `reps` launches run back to
    back between one pair of events (a decode loop's view; no event overhead)."""
    E = torch.cuda.Event
    pairs = [(E(enable_timing=True), E(enable_timing=True)) for _ in range(reps)]
    s = torch.cuda.current_stream()
    for i in range(min(len(fns), 4)):
        _check(fns[i % len(fns)]())
    torch.cuda.synchronize()
    for i in range(reps):
        pairs[i][0].record(s)
        _check(fns[i % len(fns)]())
        pairs[i][1].record(s)
    torch.cuda.synchronize()
    single = sum(a.elapsed_time(b) for a, b in pairs) / reps / 1e3
    a, b = E(enable_timing=True), E(enable_timing=True)
    a.record(s)
    for i in range(reps):
        _check(fns[i % len(fns)]())
    b.record(s)
    torch.cuda.synchronize()
    return single, a.elapsed_time(b) / reps / 1e3


def kernels(torch, prism, wl, only=None):
    dev = torch.device("cuda:0")
    L = Launcher(prism, torch.cuda.current_stream(dev).cuda_stream)

    def T(a):
        a = a.view("int16") if a.dtype.name == "uint16" else a
        return torch.from_numpy(a).to(dev)

    out = {}
    if only in (None, "w4a8"):
        c = wl.w4()
        K, N = 4096, 12288
        R = _copies(c["w4"].nbytes)
        ws = [T(c["w4"]) for _ in range(R)]
        sw = T(c["s_w"])
        for M in (1, 4, 16, 64, 512, 2048):
            # M > 64 (prefill, tiled path): the 64 seeded rows repeated (values do not change timing)
            x = T(c["x"][:M].copy() if M <= 64 else c["x"][[i % 64 for i in range(M)]])
            q = torch.empty((M, K), dtype=torch.int8, device=dev)
            sa = torch.empty((M,), dtype=torch.float32, device=dev)
            _check(L.quantize(x, q, sa)())
            y = torch.empty((M, N), dtype=torch.float32, device=dev)
            t1, t = _time_launches(torch, [L.w4a8(q, sa, w, sw, y) for w in ws], 100)
            nbytes = N * K // 2 + 4 * N + M * K + 4 * M + 4 * M * N
            out["w4a8_m%d" % M] = dict(us=t * 1e6, gbs=nbytes / t / 1e9, hbm_frac=nbytes / t / 1e9 / PEAK_HBM_GBS,
                                       tops=2 * M * N * K / t / 1e12, us_single_launch=t1 * 1e6,
                                       algorithmic_bytes=nbytes, copies=R)
        del ws
    if only in (None, "block"):
        c = wl.block()
        M, K = c["x"].shape
        N = c["w"].shape[0]
        R = _copies(c["w"].nbytes + c["d"].nbytes)
        ws = [(T(c["w"]), T(c["d"])) for _ in range(R)]
        x = T(c["x"])
        q = torch.empty((M, K), dtype=torch.int8, device=dev)
        sa = torch.empty((M,), dtype=torch.float32, device=dev)
        _check(L.quantize(x, q, sa)())
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
        t1, t = _time_launches(torch, [L.block(q, sa, w, d, y) for w, d in ws], 10)
        ops = 2 * M * N * K
        out["block_scale_m2048"] = dict(us=t * 1e6, tops=ops / t / 1e12, mfma_frac=ops / t / 1e12 / PEAK_INT8_TOPS,
                                        us_single_launch=t1 * 1e6, copies=R)
        # decode: one row through the small-M block kernel (HBM-bound: weights and scales)
        q1, sa1, y1 = q[:1].contiguous(), sa[:1].contiguous(), torch.empty((1, N), dtype=torch.float32, device=dev)
        t1, t = _time_launches(torch, [L.block(q1, sa1, w, d, y1) for w, d in ws], 50)
        nb1 = N * K + 2 * N * (K // 32) + K + 4 + 4 * N
        out["block_scale_m1"] = dict(us=t * 1e6, gbs=nb1 / t / 1e9, hbm_frac=nb1 / t / 1e9 / PEAK_HBM_GBS,
                                     us_single_launch=t1 * 1e6, algorithmic_bytes=nb1, copies=R)
        del ws
    if only in (None, "repack"):
        # Q8_0 blocks of the block-scale weight matrix (17408 x 5120): 34 bytes read and
        # 34 bytes written per 32-weight block
        N, K = 17408, 5120
        nblk = N * (K // 32)
        g = torch.Generator(device=dev).manual_seed(11)
        R = _copies(2 * 34 * nblk)
        srcs = [torch.randint(0, 256, (nblk * 34,), dtype=torch.uint8, device=dev, generator=g) for _ in range(R)]
        w = torch.empty((N, K), dtype=torch.int8, device=dev)
        d = torch.empty((N, K // 32), dtype=torch.int16, device=dev)
        t1, t = _time_launches(torch, [L.repack(b, w, d) for b in srcs], 20)
        nbytes = 2 * 34 * nblk
        out["repack_q8_0_17408x5120"] = dict(us=t * 1e6, gbs=nbytes / t / 1e9, hbm_frac=nbytes / t / 1e9 / PEAK_HBM_GBS,
                                             us_single_launch=t1 * 1e6, algorithmic_bytes=nbytes, copies=R)
        del srcs
    if only in (None, "q4k"):
        # Q4_K weights of the block-scale shape (17408 x 5120): seeded super-block bytes
        # whose d and dmin are finite binary16 values (timing only), R copies, each
        # repacked once into its planes; then the GEMM at M = 2048 and M = 1
        import numpy as np
        N, K = 17408, 5120
        nsb = N * (K // 256)
        rng = np.random.default_rng(12)
        host_blocks = rng.integers(0, 256, (nsb, 144), dtype=np.uint8)
        dd = (rng.uniform(0.5, 1.0, (nsb, 2)) * 2.0 ** rng.integers(-13, -5, (nsb, 2))).astype("<f2")
        host_blocks[:, 0:4] = dd.view(np.uint8).reshape(nsb, 4)
        blocks = torch.from_numpy(host_blocks.reshape(-1)).to(dev)
        R = _copies(N * K // 2 + nsb * 16)
        planes = [(torch.empty((N, K // 2), dtype=torch.uint8, device=dev),
                   torch.empty((N, K // 256, 16), dtype=torch.uint8, device=dev)) for _ in range(R)]
        t1, t = _time_launches(torch, [L.repack_q4k(blocks, *p) for p in planes], 20)
        nbytes = 2 * nsb * 144
        out["repack_q4_k_17408x5120"] = dict(us=t * 1e6, gbs=nbytes / t / 1e9, hbm_frac=nbytes / t / 1e9 / PEAK_HBM_GBS,
                                             us_single_launch=t1 * 1e6, algorithmic_bytes=nbytes)
        torch.cuda.synchronize()
        del blocks
        xb = wl.block()["x"]
        for M in (2048, 1):
            x = torch.from_numpy(xb[:M].copy()).to(dev)
            q = torch.empty((M, K), dtype=torch.int8, device=dev)
            sa = torch.empty((M,), dtype=torch.float32, device=dev)
            _check(L.quantize(x, q, sa)())
            y = torch.empty((M, N), dtype=torch.float32, device=dev)
            t1, t = _time_launches(torch, [L.q4k(q, sa, *p, y) for p in planes], 10 if M > 1 else 50)
            ops = 2 * M * N * K
            nb = N * K // 2 + nsb * 16 + M * K + 4 * M + 4 * M * N   # packed codes, headers, q, s_a, y
            out["q4k_m%d" % M] = dict(us=t * 1e6, tops=ops / t / 1e12, mfma_frac=ops / t / 1e12 / PEAK_INT8_TOPS,
                                      gbs=nb / t / 1e9, hbm_frac=nb / t / 1e9 / PEAK_HBM_GBS,
                                      us_single_launch=t1 * 1e6, copies=R, algorithmic_bytes=nb)
        del planes
    if only in (None, "decode"):
        # One activation row (decode) through the two projections of the step.
        for name, c in (("proj_up", wl.proj_up()), ("proj_down", wl.proj_down())):
            N, K = c["w"].shape
            R = _copies(c["w"].nbytes)
            ws = [T(c["w"]) for _ in range(R)]
            sw = T(c["s_w"])
            x = T(c["x"][:1].copy())
            q = torch.empty((1, K), dtype=torch.int8, device=dev)
            sa = torch.empty((1,), dtype=torch.float32, device=dev)
            _check(L.quantize(x, q, sa)())
            y = torch.empty((1, N), dtype=torch.float32, device=dev)
            t1, t = _time_launches(torch, [L.w8a8(q, sa, w, sw, y) for w in ws], 100)
            nbytes = N * K + 4 * N + K + 4 + 4 * N
            out["decode_m1_" + name] = dict(us=t * 1e6, gbs=nbytes / t / 1e9, hbm_frac=nbytes / t / 1e9 / PEAK_HBM_GBS,
                                            us_single_launch=t1 * 1e6, algorithmic_bytes=nbytes, copies=R)
            # the whole decode step of this projection: quantize x, then the GEMM
            pairs = []
            for w in ws:
                fq, fg = L.quantize(x, q, sa), L.w8a8(q, sa, w, sw, y)
                pairs.append(lambda fq=fq, fg=fg: fq() or fg())
            _, t2 = _time_launches(torch, pairs, 100)
            _, t3 = _time_launches(torch, [L.quantize_w8a8(x, q, sa, w, sw, y) for w in ws], 100)
            nbytes_x = nbytes - K - 4 + 4 * K   # x read as fp32 instead of the codes
            out["decode_m1_" + name].update(quantize_then_gemm_us=t2 * 1e6, fused_quantize_gemm_us=t3 * 1e6,
                                            fused_hbm_frac=nbytes_x / t3 / 1e9 / PEAK_HBM_GBS)
            # a few rows (batched decode): two launches against the one-launch call
            for M in (2, 4, 16):
                xm = T(c["x"][:M].copy())
                qm = torch.empty((M, K), dtype=torch.int8, device=dev)
                sam = torch.empty((M,), dtype=torch.float32, device=dev)
                ym = torch.empty((M, N), dtype=torch.float32, device=dev)
                pairs = []
                for w in ws:
                    fq, fg = L.quantize(xm, qm, sam), L.w8a8(qm, sam, w, sw, ym)
                    pairs.append(lambda fq=fq, fg=fg: fq() or fg())
                _, t2 = _time_launches(torch, pairs, 100)
                _, t3 = _time_launches(torch, [L.quantize_w8a8(xm, qm, sam, w, sw, ym) for w in ws], 100)
                nb = N * K + 4 * N + 4 * M * K + M * K + 4 * M + 4 * M * N   # w, s_w, x, q, scale, y
                out["decode_m%d_%s" % (M, name)] = dict(quantize_then_gemm_us=t2 * 1e6, fused_quantize_gemm_us=t3 * 1e6,
                                                        fused_hbm_frac=nb / t3 / 1e9 / PEAK_HBM_GBS,
                                                        algorithmic_bytes=nb, copies=R)
            del ws
    if only in (None, "vendor"):
        # Context: the vendor int8 GEMM (hipBLASLt through torch._int_mm) on the
        # same shapes, int32 output only (no activation or weight scales, so it
        # does less work than prism_gemm_w8a8); weights rotated as above.
        g = torch.Generator(device=dev)
        g.manual_seed(11)
        for name, (M, N, K) in (("proj_up", (512, 9728, 2560)), ("proj_down", (512, 2560, 9728)),
                                ("stress_m8192", (8192, 5120, 5120))):
            R = _copies(N * K)
            q = torch.randint(-127, 128, (M, K), dtype=torch.int8, device=dev, generator=g)
            wts = [torch.randint(-127, 128, (N, K), dtype=torch.int8, device=dev, generator=g) for _ in range(R)]
            try:
                def mm(wt):
                    return lambda: (torch._int_mm(q, wt.t()), 0)[1]
                t1, t = _time_launches(torch, [mm(wt) for wt in wts], 20)
                out["vendor_int_mm_" + name] = dict(us=t * 1e6, tops=2 * M * N * K / t / 1e12,
                                                    mfma_frac=2 * M * N * K / t / 1e12 / PEAK_INT8_TOPS,
                                                    us_single_launch=t1 * 1e6, copies=R)
            except RuntimeError as e:   # not every torch build exposes an int8 GEMM
                out["vendor_int_mm_" + name] = dict(error=str(e)[:120])
            del wts
    if only in (None, "peaks"):
        # What this GPU reaches on the two resources, with the library's own
        # measurement kernels: int8 MFMA on registers (no memory traffic) at 1,
        # 2 and 4 waves per SIMD, and a plain once-through read of 25.2 MB
        # (the size of one projection's int8 weights; copies rotated so that
        # nothing is cached) and of 1 GiB.
        ncu = torch.cuda.get_device_properties(dev).multi_processor_count
        peaks = {}
        for wps in (1, 2, 4):
            iters = 8192 // wps
            outp = torch.empty((2 * ncu * 128 * wps,), dtype=torch.int32, device=dev)
            f = L.lib.prism_peak_mfma
            args = (iters, wps, 1, L.p(outp), L.stream)
            t1, t = _time_launches(torch, [lambda: f(*args)], 5)
            ops = 2 * ncu * 2 * wps * iters * 16 * 65536
            peaks["mfma_i8_%dw_per_simd" % wps] = dict(us=t * 1e6, tops=ops / t / 1e12,
                                                       mfma_frac=ops / t / 1e12 / PEAK_INT8_TOPS)
        # The block-scale fold on registers: ns per 32-k block of one 32 x 32
        # tile per SIMD (two waves per SIMD), int8 MFMA + convert + fmaf
        # against f16 MFMA pairs + fmaf, and each part alone.
        outf = torch.empty((ncu * 512,), dtype=torch.float32, device=dev)
        iters = 4000
        for mode, name in enumerate(prism.FOLD_MODES):
            f = L.lib.prism_peak_fold
            args = (mode, iters, L.p(outf), L.stream)
            t1, t = _time_launches(torch, [lambda: f(*args)], 5)
            peaks["fold_" + name] = dict(us=t * 1e6, ns_per_tile_block_per_simd=t * 1e9 / (2 * iters * prism.FOLD_TILES))
        parts = torch.empty((4096,), dtype=torch.int32, device=dev)
        for name, nbytes in (("read_25.2MB", 9728 * 2560), ("read_1GiB", 1 << 30)):
            R = _copies(nbytes)
            bufs = [torch.empty((nbytes,), dtype=torch.uint8, device=dev).fill_(i) for i in range(R)]
            f = L.lib.prism_peak_read
            fns = [(lambda b=b: f(L.p(b), nbytes, L.p(parts), L.stream)) for b in bufs]
            t1, t = _time_launches(torch, fns, max(10, 2 * R))
            peaks[name] = dict(us=t * 1e6, gbs=nbytes / t / 1e9, hbm_frac=nbytes / t / 1e9 / PEAK_HBM_GBS,
                               us_single_launch=t1 * 1e6, gbs_single_launch=nbytes / t1 / 1e9, copies=R)
            del bufs
        out["peaks"] = peaks
        # The block fold's floor from the measurement kernel: per SIMD, each 32-k
        # block of a 32 x 32 tile costs one int8 MFMA, 16 converts and 16 fmaf
        # (block-scale), plus 16 more fmaf for the Q4_K min term; the two
        # tiled GEMMs at M = 2048 do (M/32)(N/32)(K/32) / 1024 of them per SIMD.
        ns_fold = peaks["fold_i8_mfma_cvt_fold"]["ns_per_tile_block_per_simd"]
        ns_fma = peaks["fold_fold_only"]["ns_per_tile_block_per_simd"]
        per_simd = (2048 // 32) * (17408 // 32) * (5120 // 32) / 1024
        for name, ns in (("block_scale_m2048", ns_fold), ("q4k_m2048", ns_fold + ns_fma)):
            if name in out:
                floor_us = per_simd * ns / 1e3
                out[name].update(fold_floor_us=floor_us, fold_floor_frac=floor_us / out[name]["us"])
    if only == "sweep":
        # Not in the default run: the per-channel W8A8 GEMM across M at
        # N = K = 5120 (the plain call's own kernel choice at each M), next to
        # the vendor int8 GEMM on the same inputs (int32 output only); weights
        # rotated as above.  Inputs are seeded int8 codes (values do not change
        # the kernels' timing much; the stress workload covers real activations).
        g = torch.Generator(device=dev)
        g.manual_seed(12)
        N = K = 5120
        R = _copies(N * K)
        wts = [torch.randint(-127, 128, (N, K), dtype=torch.int8, device=dev, generator=g) for _ in range(R)]
        sw = torch.rand((N,), device=dev, generator=g) * 0.01
        for M in (1, 4, 16, 64, 128, 256, 512, 1024, 2048, 4096, 8192):
            q = torch.randint(-127, 128, (M, K), dtype=torch.int8, device=dev, generator=g)
            sa = torch.rand((M,), device=dev, generator=g) * 0.01
            y = torch.empty((M, N), dtype=torch.float32, device=dev)
            reps = 100 if M <= 256 else 20
            t1, t = _time_launches(torch, [L.w8a8(q, sa, wt, sw, y) for wt in wts], reps)
            nbytes = N * K + 4 * N + M * K + 4 * M + 4 * M * N
            rec = dict(us=t * 1e6, tops=2 * M * N * K / t / 1e12, mfma_frac=2 * M * N * K / t / 1e12 / PEAK_INT8_TOPS,
                       gbs=nbytes / t / 1e9, hbm_frac=nbytes / t / 1e9 / PEAK_HBM_GBS, copies=R)
            try:
                def mm(wt):
                    return lambda: (torch._int_mm(q, wt.t()), 0)[1]
                _, tv = _time_launches(torch, [mm(wt) for wt in wts], reps)
                rec.update(vendor_int_mm_us=tv * 1e6, vendor_over_prism=tv / t)
            except RuntimeError as e:   # the vendor GEMM takes M > 16 only on some builds
                rec.update(vendor_int_mm_error=str(e)[:80])
            out["sweep_w8a8_5120x5120_m%d" % M] = rec
        del wts
    if only in (None, "proj"):
        out["step_proj_m512"] = proj_step(torch, prism, wl)
    if only in (None, "stress"):
        st = wl.stress()
        R = _copies(st["w"].nbytes)
        ws = [T(st["w"]) for _ in range(R)]   # rotated, so that no launch finds W in the MALL
        sw = T(st["s_w"])
        K = N = 5120
        x_over, _ = wl.stress_overwrite(st)
        # M = 8192 is also the headline step; here its GEMM is timed on its own
        # (launches back to back, weights rotated), next to the static quantizer
        for M, xa in ((8192, x_over), (1, st["x_probe"][:1].copy())):
            x = T(xa)
            q = torch.empty((M, K), dtype=torch.int8, device=dev)
            sa = torch.empty((M,), dtype=torch.float32, device=dev)
            _, tq = _time_launches(torch, [L.quantize(x, q, sa)], 20)
            _, tqs = _time_launches(torch, [L.quantize_static(x, q, sa, 0.03)], 20)
            _check(L.quantize(x, q, sa)())   # the GEMM below runs on the per-row codes
            y = torch.empty((M, N), dtype=torch.float32, device=dev)
            t1, t = _time_launches(torch, [L.w8a8(q, sa, w, sw, y) for w in ws], 20 if M > 1 else 100)
            nbytes = N * K + 4 * N + M * K + 4 * M + 4 * M * N
            out["stress_m%d" % M] = dict(copies=R, us=t * 1e6, tops=2 * M * N * K / t / 1e12,
                                         mfma_frac=2 * M * N * K / t / 1e12 / PEAK_INT8_TOPS,
                                         gbs=nbytes / t / 1e9, hbm_frac=nbytes / t / 1e9 / PEAK_HBM_GBS,
                                         quantize_us=tq * 1e6, us_single_launch=t1 * 1e6,
                                         quantize_gbs=(5 * M * K + 4 * M) / tq / 1e9,
                                         quantize_static_us=tqs * 1e6,
                                         quantize_static_gbs=(5 * M * K + 4 * M) / tqs / 1e9)
    return out


# ------------------------------------------------------------------ CPU oracle

def cpu_baseline(np, oracle, case, gpu_out, budget_s=12.0):
    """The oracle, as it stands, on the host cores, on the headline step's work
    (quantize rows + W8A8 GEMM): full steps repeated until the budget is spent,
    or the first rows of one step if a full step would take far longer.  The
    sampled rows are compared bit for bit with the GPU's outputs."""
    x, w, s_w = case["x"], case["w"], case["s_w"]
    M, K = x.shape
    N = w.shape[0]
    t0 = time.perf_counter()
    oracle.gemm_w8a8(*oracle.quantize_rows(x[:64]), w, s_w)
    est_full = (time.perf_counter() - t0) * M / 64
    rows = M if est_full <= 2 * budget_s else max(64, int(M * budget_s / est_full) // 64 * 64)
    reps, out = 0, None
    t0 = time.perf_counter()
    while reps == 0 or (time.perf_counter() - t0 < budget_s and rows == M):
        q, s = oracle.quantize_rows(x[:rows])
        y, _ = oracle.gemm_w8a8(q, s, w, s_w)
        out = (q, s, y)
        reps += 1
    dt = time.perf_counter() - t0
    ops = reps * 2 * rows * N * K
    gq, gs, gy = gpu_out
    q, s, y = out
    exact = bool(np.array_equal(gq[:rows], q) and np.array_equal(gs[:rows].view(np.uint32), s.view(np.uint32))
                 and np.array_equal(gy[:rows].view(np.uint32), y.view(np.uint32)))
    sample = ("%d full step(s) (quantize + GEMM, M=%d, K=%d, N=%d)" % (reps, M, K, N) if rows == M else
              "rows 0..%d of one step (quantize + GEMM, K=%d, N=%d)" % (rows - 1, K, N))
    return dict(value=ops / dt / 1e12, unit="TOPS", cores=oracle.max_threads(), kind="oracle", sample=sample,
                seconds=dt, cpu=_cpu_model(), nproc=os.cpu_count(), compiler="gcc " + " ".join(oracle.CFLAGS)), exact


def _cpu_model():
    """The host CPU's model name (from /proc/cpuinfo where there is one)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def main():
    args = _args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from exact_int8_gemm_amd import prism
    from exact_int8_gemm_amd import workloads as wl

    if args.calib_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.only is not None and args.only != "step":
        print(json.dumps(kernels(torch, prism, wl, only=args.only)))
        return
    # The per-kernel measurements of the default run go between the headline's
    # setup (inputs generated and copied to the GPU, about a second of host
    # work) and its warm-up steps: they also bring a GPU that has been idle to
    # its steady clocks, which takes some tens of milliseconds of load (the
    # first ~40 steps of the stress step run 10-15% slower than the rest on
    # MI355X).  The W warm-up steps and the K timed steps are exactly as
    # requested.
    def other_kernels():
        if args.only is None and not args.no_kernels:
            k = kernels(torch, prism, wl)
            print("kernel measurements done", file=sys.stderr, flush=True)
            return k
        return None
    h = headline(torch, prism, wl, args, before_timing=other_kernels)
    k = h["extra"]
    print("headline step done: %.1f us per step" % (h["ms_per_step"] * 1e3), file=sys.stderr, flush=True)
    rec = {
        "metric": METRIC, "value": h["value"], "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": h["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int8", "data": "synthetic",
        "config": {"workload": "batch-invariance stress batch, W8A8 per-channel: quantize rows of X [8192 x 5120] "
                               "(64 probe rows among N(0,1) rows) + GEMM with W [5120 x 5120]",
                   "M": h["M"], "K": h["K"], "N": h["N"], "rotated_input_copies": h["R"],
                   "parallelism": "single GPU"},
        "roofline": h["roofline"],
    }
    if args.only is None and not args.no_cpu:
        import oracle
        o = h["outputs"][0]
        cb, exact = cpu_baseline(np, oracle, h["case"], (o[0].cpu().numpy(), o[1].cpu().numpy(), o[2].cpu().numpy()))
        rec["cpu_baseline"] = cb
        rec["bit_exact_vs_oracle"] = exact
        print("cpu baseline done", file=sys.stderr, flush=True)
    if k is not None:
        rec["kernels"] = k
        # the two regimes of the measurement targets, side by side
        small = {n: k[n]["hbm_frac"] for n in ("w4a8_m1", "w4a8_m4", "w4a8_m16", "stress_m1", "decode_m1_proj_up",
                                               "decode_m1_proj_down", "block_scale_m1", "q4k_m1") if n in k}
        rec["targets"] = {"m_ge_2048_mfma_frac": {"stress_m8192 (headline GEMM)": h["roofline"]["frac"],
                                                  "block_scale_m2048": k.get("block_scale_m2048", {}).get("mfma_frac"),
                                                  "w4a8_m2048": k.get("w4a8_m2048", {}).get("mfma_frac"),
                                                  "q4k_m2048": k.get("q4k_m2048", {}).get("mfma_frac")},
                          "m_le_16_hbm_frac": small}
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
