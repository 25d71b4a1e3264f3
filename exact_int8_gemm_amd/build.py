"""Ahead-of-time build of libprism.so for gfx950 (MI355X) with hipcc.

Each source is compiled to an object in ``_build/`` (in parallel), then the
objects are linked into ``exact_int8_gemm_amd/libprism.so`` in-tree.

Flags that define results, not only speed:
  -ffp-contract=off                           no fused multiply-add except the
                                              fmaf() the block epilogue asks for
  -fhip-fp32-correctly-rounded-divide-sqrt    IEEE division in the quantizer
  -fno-gpu-flush-denormals-to-zero            fp32 subnormals kept
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                              no packed fp32 instructions
"""
from __future__ import annotations

import hashlib
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libprism.so")

SOURCES = ["quantize.hip", "gemm_small.hip", "gemm_tiled.hip", "repack.hip", "peaks.hip", "prism_abi.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function", "-Werror=inline-asm",
    "-ffp-contract=off", "-fno-fast-math",
]
DEVICE = [
    "--offload-arch=" + ARCH,
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources():
    return [os.path.join(CSRC, s) for s in SOURCES]


def source_hash() -> str:
    """sha256 (hex, 32 digits) of every file under csrc/, of include/prism.h and of
    the compile flags.  It is compiled into the library (prism_build_id), so a
    binary can be matched against the sources it is meant to come from."""
    h = hashlib.sha256()
    files = sorted(os.listdir(CSRC))
    for name in files:
        path = os.path.join(CSRC, name)
        if os.path.isfile(path):
            h.update(name.encode() + b"\0")
            with open(path, "rb") as f:
                h.update(f.read())
    with open(os.path.join(ROOT, "include", "prism.h"), "rb") as f:
        h.update(b"prism.h\0" + f.read())
    h.update(" ".join(COMMON + DEVICE).encode())
    return h.hexdigest()[:32]


def _compile_cmd(src, obj, build_id="0" * 32):
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    return [HIPCC, *lang, *COMMON, *DEVICE, "-I", os.path.join(ROOT, "include"),
            '-DPRISM_BUILD_ID="%s"' % build_id, "-c", src, "-o", obj]


def build_library(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libprism.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    build_id = source_hash()
    procs = []
    objs = []
    for src in sources():
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        objs.append(obj)
        cmd = _compile_cmd(src, obj, build_id)
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the packed-fp32 feature and says so: harmless
        lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln]
        if lines and (verbose or p.returncode):
            print("\n".join(lines), file=sys.stderr)
        if p.returncode:
            failed.append(src)
    if failed:
        raise RuntimeError("hipcc failed for: " + ", ".join(os.path.basename(f) for f in failed))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
