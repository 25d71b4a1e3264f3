"""The C ABI library loads, exports what include/prism.h declares, and rejects
invalid calls before any HIP call (runs without a GPU).

The validation calls pass fake pointers, so they run in a child process in
which no HIP device is visible: even a validation bug could then never reach
a kernel launch.  The child asks the HIP runtime for its device count first
and makes no call at all if it sees a device.
"""
import json
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "prism.h")
LIB = os.path.join(ROOT, "exact_int8_gemm_amd", "libprism.so")


def _header():
    return open(HEADER).read()


def _declared_functions():
    return re.findall(r"^\s*(?:int|const char\*)\s+(prism_\w+)\s*\(", _header(), flags=re.M)


def _defines():
    return {k: int(v) for k, v in re.findall(r"#define\s+(PRISM_\w+)\s+\(?(-?\d+)\)?", _header())}


@pytest.fixture(scope="module")
def built():
    if not os.path.exists(LIB):
        sys.path.insert(0, ROOT)
        from exact_int8_gemm_amd import build
        build.build_library()
    return LIB


def test_header_declares_every_call():
    names = set(_declared_functions())
    assert {"prism_quantize_rows", "prism_quantize_rows_static", "prism_repack_q8_0", "prism_gemm_w8a8",
            "prism_gemm_w8a8_blockscale", "prism_gemm_w4a8", "prism_gemm_w8a8_variant", "prism_gemm_w4a8_variant",
            "prism_repack_q4_k", "prism_gemm_w4a8_q4k", "prism_quantize_gemm_w8a8",
            "prism_peak_mfma", "prism_peak_read", "prism_peak_fold", "prism_abi_version", "prism_build_id", "prism_status_string"} <= names


def test_library_exports_every_declared_symbol(built):
    out = subprocess.run(["nm", "-D", "--defined-only", built], capture_output=True, text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    for name in _declared_functions():
        assert name in exported, name


def test_binding_constants_match_header():
    sys.path.insert(0, ROOT)
    from exact_int8_gemm_amd import prism
    d = _defines()
    assert d["PRISM_ABI_VERSION"] == prism.ABI_VERSION
    assert d["PRISM_K_MAX"] == prism.K_MAX
    # the K bound keeps every exact sum inside int32 even for -128 * -128 products
    assert d["PRISM_K_MAX"] * 128 * 128 < 2 ** 31
    assert d["PRISM_K_MAX"] % 32 == 0


_CHILD = r"""
import ctypes, json, sys
lib = ctypes.CDLL(sys.argv[1])
# The calls below pass fake device addresses.  Refuse to make any of them if the
# HIP runtime that libprism loaded can see a device (the parent hides devices
# through the environment; this checks that the hiding took effect).
hip = ctypes.CDLL("libamdhip64.so.7")
count = ctypes.c_int(0)
if hip.hipGetDeviceCount(ctypes.byref(count)) == 0 and count.value > 0:
    print(json.dumps({"device_visible": count.value}))
    sys.exit(0)
p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
lib.prism_abi_version.restype = i32
lib.prism_status_string.restype = ctypes.c_char_p
lib.prism_status_string.argtypes = [i32]
lib.prism_quantize_rows.restype = i32
lib.prism_quantize_rows.argtypes = [p, p, p, i64, i64, p]
lib.prism_quantize_rows_static.restype = i32
lib.prism_quantize_rows_static.argtypes = [p, p, p, ctypes.c_float, i64, i64, p]
lib.prism_repack_q8_0.restype = i32
lib.prism_repack_q8_0.argtypes = [p, p, p, i64, i64, p]
lib.prism_repack_q4_k.restype = i32
lib.prism_repack_q4_k.argtypes = [p, p, p, i64, i64, p]
lib.prism_gemm_w4a8_q4k.restype = i32
lib.prism_gemm_w4a8_q4k.argtypes = [p, p, p, p, p, i64, i64, i64, p]
lib.prism_quantize_gemm_w8a8.restype = i32
lib.prism_quantize_gemm_w8a8.argtypes = [p, p, p, p, p, p, p, i64, i64, i64, p]
for n in ("prism_gemm_w8a8_variant", "prism_gemm_w4a8_variant"):
    getattr(lib, n).restype = i32
    getattr(lib, n).argtypes = [p, p, p, p, p, p, i64, i64, i64, i32, p]
for n in ("prism_gemm_w8a8", "prism_gemm_w8a8_blockscale", "prism_gemm_w4a8"):
    getattr(lib, n).restype = i32
    getattr(lib, n).argtypes = [p, p, p, p, p, p, i64, i64, i64, p]
lib.prism_peak_mfma.restype = i32
lib.prism_peak_mfma.argtypes = [i64, i32, i32, p, p]
lib.prism_peak_read.restype = i32
lib.prism_peak_read.argtypes = [p, i64, p, p]
lib.prism_peak_fold.restype = i32
lib.prism_peak_fold.argtypes = [i32, i64, p, p]
A = 0x7f0000000000          # 256-byte aligned fake address, never dereferenced
res = {"version": lib.prism_abi_version(),
       "strings": {str(s): lib.prism_status_string(s).decode() for s in (0, -1, -2, -3, -4, 7)}}
cases = json.loads(sys.argv[2])
out = []
for fn, args in cases:
    out.append(getattr(lib, fn)(*[None if a is None else a for a in args]))
res["status"] = out
print(json.dumps(res))
"""

OK, INVALID, ALIGN, UNSUP = 0, -1, -2, -3
A = 0x7F0000000000


def _g(q=A, sa=A, w=A, sw=A, y=A, acc=None, M=4, N=16, K=64):
    return [q, sa, w, sw, y, acc, M, N, K, None]


# (function, args, expected status); every non-OK case is invalid before any HIP call
CASES = [
    ("prism_quantize_rows", [A, A, A, 0, 64, None], OK),            # M = 0: no-op
    ("prism_quantize_rows", [None, None, None, 0, 0, None], OK),    # M = 0 with nothing at all
    ("prism_quantize_rows", [A, A, A, -1, 64, None], INVALID),
    ("prism_quantize_rows", [A, A, A, 4, -16, None], INVALID),
    ("prism_quantize_rows", [A, A, A, 4, 0, None], INVALID),
    ("prism_quantize_rows", [None, A, A, 4, 64, None], INVALID),
    ("prism_quantize_rows", [A, None, A, 4, 64, None], INVALID),
    ("prism_quantize_rows", [A, A, None, 4, 64, None], INVALID),
    ("prism_quantize_rows", [A, A, A, 4, 40, None], ALIGN),          # K % 16
    ("prism_quantize_rows", [A + 4, A, A, 4, 64, None], ALIGN),
    ("prism_quantize_rows", [A, A + 8, A, 4, 64, None], ALIGN),
    ("prism_quantize_rows", [A, A, A + 2, 4, 64, None], ALIGN),
]
_QS = "prism_quantize_rows_static"
CASES += [
    (_QS, [A, A, A, 1.0, 0, 64, None], OK),             # M = 0: no-op
    (_QS, [None, None, None, 0.5, 0, 0, None], OK),
    (_QS, [A, A, A, 0.0, 4, 64, None], INVALID),        # the scale must be finite and > 0
    (_QS, [A, A, A, -1.0, 4, 64, None], INVALID),
    (_QS, [A, A, A, float("inf"), 4, 64, None], INVALID),
    (_QS, [A, A, A, float("nan"), 4, 64, None], INVALID),
    (_QS, [A, A, A, float("nan"), 0, 64, None], INVALID),  # checked even when M = 0
    (_QS, [A, A, A, 1.0, -1, 64, None], INVALID),
    (_QS, [A, A, A, 1.0, 4, -16, None], INVALID),
    (_QS, [A, A, A, 1.0, 4, 0, None], INVALID),
    (_QS, [None, A, A, 1.0, 4, 64, None], INVALID),
    (_QS, [A, None, A, 1.0, 4, 64, None], INVALID),
    (_QS, [A, A, None, 1.0, 4, 64, None], INVALID),
    (_QS, [A, A, A, 1.0, 4, 40, None], ALIGN),
    (_QS, [A + 4, A, A, 1.0, 4, 64, None], ALIGN),
    (_QS, [A, A + 8, A, 1.0, 4, 64, None], ALIGN),
    (_QS, [A, A, A + 2, 1.0, 4, 64, None], ALIGN),
]
_RP = "prism_repack_q8_0"
CASES += [
    (_RP, [A, A, A, 0, 64, None], OK),                  # N = 0: no-op
    (_RP, [None, None, None, 0, 0, None], OK),
    (_RP, [A, A, A, -1, 64, None], INVALID),
    (_RP, [A, A, A, 4, -32, None], INVALID),
    (_RP, [A, A, A, 4, 0, None], INVALID),
    (_RP, [A, A, A, 1 << 31, 64, None], INVALID),
    (_RP, [None, A, A, 4, 64, None], INVALID),
    (_RP, [A, None, A, 4, 64, None], INVALID),
    (_RP, [A, A, None, 4, 64, None], INVALID),
    (_RP, [A, A, A, 4, 48, None], ALIGN),               # K % 32
    (_RP, [A + 4, A, A, 4, 64, None], ALIGN),
    (_RP, [A, A + 8, A, 4, 64, None], ALIGN),
    (_RP, [A, A, A + 1, 4, 64, None], ALIGN),
]
_RK = "prism_repack_q4_k"
CASES += [
    (_RK, [A, A, A, 0, 256, None], OK),
    (_RK, [A, A, A, -1, 256, None], INVALID),
    (_RK, [A, A, A, 4, 0, None], INVALID),
    (_RK, [None, A, A, 4, 256, None], INVALID),
    (_RK, [A, None, A, 4, 256, None], INVALID),
    (_RK, [A, A, None, 4, 256, None], INVALID),
    (_RK, [A, A, A, 4, 288, None], ALIGN),          # K % 256
    (_RK, [A + 8, A, A, 4, 256, None], ALIGN),
    (_RK, [A, A + 8, A, 4, 256, None], ALIGN),
    (_RK, [A, A, A + 8, 4, 256, None], ALIGN),
]
_GK = "prism_gemm_w4a8_q4k"


def _k(q=A, sa=A, w4=A, hdr=A, y=A, M=4, N=16, K=256):
    return [q, sa, w4, hdr, y, M, N, K, None]


CASES += [
    (_GK, _k(M=0), OK),
    (_GK, _k(M=-1), INVALID),
    (_GK, _k(K=0), INVALID),
    (_GK, _k(hdr=None), INVALID),
    (_GK, _k(w4=None), INVALID),
    (_GK, _k(q=None), INVALID),
    (_GK, _k(K=48), ALIGN),
    (_GK, _k(K=288), ALIGN),       # whole super-blocks only
    (_GK, _k(hdr=A + 8), ALIGN),
    (_GK, _k(w4=A + 8), ALIGN),
    (_GK, _k(y=A + 2), ALIGN),
]


_QG = "prism_quantize_gemm_w8a8"


def _qg(x=A, q=A, scale=A, w=A, sw=A, y=A, acc=None, M=1, N=16, K=64):
    return [x, q, scale, w, sw, y, acc, M, N, K, None]


CASES += [
    (_QG, _qg(M=0), OK),
    (_QG, _qg(None, None, None, None, None, None, None, 0, 16, 64), OK),
    (_QG, _qg(M=-1), INVALID),
    (_QG, _qg(N=0), INVALID),
    (_QG, _qg(K=0), INVALID),
    (_QG, _qg(K=131040 + 16), INVALID),
    (_QG, _qg(x=None), INVALID),
    (_QG, _qg(q=None), INVALID),
    (_QG, _qg(scale=None), INVALID),
    (_QG, _qg(w=None), INVALID),
    (_QG, _qg(sw=None), INVALID),
    (_QG, _qg(y=None), INVALID),
    (_QG, _qg(K=40), ALIGN),
    (_QG, _qg(x=A + 4), ALIGN),
    (_QG, _qg(q=A + 8), ALIGN),
    (_QG, _qg(scale=A + 2), ALIGN),
    (_QG, _qg(w=A + 8), ALIGN),
    (_QG, _qg(sw=A + 2), ALIGN),
    (_QG, _qg(y=A + 2), ALIGN),
    (_QG, _qg(acc=A + 2), ALIGN),
]


def _v(variant, **kw):
    a = _g(**kw)
    return a[:9] + [variant, None]


for fn in ("prism_gemm_w8a8_variant", "prism_gemm_w4a8_variant"):
    CASES += [
        (fn, _v(-1), INVALID),                 # unknown variant: refused before anything else
        (fn, _v(27), INVALID),
        (fn, _v(27, M=0), INVALID),
        (fn, _v(0, M=0), OK),
        (fn, _v(3, M=0), OK),
        (fn, _v(0, q=None), INVALID),
        (fn, _v(9, K=0), INVALID),
        (fn, _v(9, K=40), ALIGN),
        (fn, _v(9, y=A + 2), ALIGN),
        (fn, _v(9, sw=A + 2), ALIGN),
    ]
for fn, kmul in (("prism_gemm_w8a8", 16), ("prism_gemm_w4a8", 32), ("prism_gemm_w8a8_blockscale", 32)):
    CASES += [
        (fn, _g(M=0), OK),
        (fn, _g(None, None, None, None, None, None, 0, 16, 64), OK),
        (fn, _g(M=-1), INVALID),
        (fn, _g(N=-1), INVALID),
        (fn, _g(K=-32), INVALID),
        (fn, _g(M=-1, N=0, K=0), INVALID),
        (fn, _g(N=0), INVALID),
        (fn, _g(K=0), INVALID),
        (fn, _g(K=131040 + 32), INVALID),
        (fn, _g(K=1 << 40), INVALID),
        (fn, _g(M=1 << 31), INVALID),
        (fn, _g(N=1 << 31), INVALID),
        (fn, _g(q=None), INVALID),
        (fn, _g(sa=None), INVALID),
        (fn, _g(w=None), INVALID),
        (fn, _g(sw=None), INVALID),
        (fn, _g(y=None), INVALID),
        (fn, _g(K=kmul + 8), ALIGN),
        (fn, _g(q=A + 8), ALIGN),
        (fn, _g(w=A + 4), ALIGN),
        (fn, _g(sa=A + 2), ALIGN),
        (fn, _g(y=A + 1), ALIGN),
        (fn, _g(acc=A + 2), ALIGN),
    ]
    if kmul == 32:
        CASES.append((fn, _g(K=48), ALIGN))
CASES += [
    ("prism_peak_mfma", [0, 2, 0, A, None], INVALID),            # iters >= 1
    ("prism_peak_mfma", [(1 << 24) + 1, 2, 0, A, None], INVALID),
    ("prism_peak_mfma", [10, 3, 0, A, None], INVALID),           # waves per SIMD in {1, 2, 4}
    ("prism_peak_mfma", [10, 0, 0, A, None], INVALID),
    ("prism_peak_mfma", [10, 2, -1, A, None], INVALID),
    ("prism_peak_mfma", [10, 2, 0, None, None], INVALID),
    ("prism_peak_mfma", [10, 2, 0, A + 2, None], ALIGN),
    ("prism_peak_read", [A, 0, A, None], INVALID),
    ("prism_peak_read", [A, -16, A, None], INVALID),
    ("prism_peak_read", [None, 64, A, None], INVALID),
    ("prism_peak_read", [A, 64, None, None], INVALID),
    ("prism_peak_read", [A, (1 << 40) + 16, A, None], INVALID),
    ("prism_peak_read", [A, 40, A, None], ALIGN),                # bytes % 16
    ("prism_peak_read", [A + 8, 64, A, None], ALIGN),
    ("prism_peak_read", [A, 64, A + 1, None], ALIGN),
    ("prism_peak_fold", [-1, 10, A, None], INVALID),             # mode in 0..4
    ("prism_peak_fold", [5, 10, A, None], INVALID),
    ("prism_peak_fold", [0, 0, A, None], INVALID),               # iters in [1, 2^20]
    ("prism_peak_fold", [0, (1 << 20) + 1, A, None], INVALID),
    ("prism_peak_fold", [0, 10, None, None], INVALID),
    ("prism_peak_fold", [1, 10, A + 2, None], ALIGN),
]
CASES.append(("prism_gemm_w8a8", _g(sw=A + 2), ALIGN))
CASES.append(("prism_gemm_w4a8", _g(sw=A + 1), ALIGN))
CASES.append(("prism_gemm_w8a8_blockscale", _g(sw=A + 1), ALIGN))   # d is 2-byte data


@pytest.fixture(scope="module")
def child_results(built):
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", CUDA_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1")
    payload = json.dumps([[fn, args] for fn, args, _ in CASES])
    out = subprocess.run([sys.executable, "-c", _CHILD, built, payload], env=env, capture_output=True, text=True,
                         timeout=120)
    assert out.returncode == 0, out.stderr
    res = json.loads(out.stdout.strip().splitlines()[-1])
    if "device_visible" in res:
        pytest.skip("a HIP device is visible despite HIP_VISIBLE_DEVICES=-1: fake-pointer calls not made")
    return res


def test_abi_version(child_results):
    assert child_results["version"] == _defines()["PRISM_ABI_VERSION"]


def test_status_strings(child_results):
    s = child_results["strings"]
    assert s["0"] == "ok"
    texts = [s[k] for k in ("-1", "-2", "-3", "-4")]
    assert all(texts) and len(set(texts)) == 4
    assert s["7"] == "unknown status"


@pytest.mark.parametrize("i", range(len(CASES)))
def test_validation(child_results, i):
    fn, args, expect = CASES[i]
    assert child_results["status"][i] == expect, (fn, args)


def test_valid_call_without_a_device_is_unsupported(built):
    """Valid arguments with no visible device: the device check answers, nothing launches."""
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", CUDA_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1")
    payload = json.dumps([["prism_gemm_w8a8", _g()], ["prism_quantize_rows", [A, A, A, 4, 64, None]],
                          ["prism_quantize_rows_static", [A, A, A, 0.25, 4, 64, None]],
                          ["prism_repack_q8_0", [A, A, A, 4, 64, None]],
                          ["prism_gemm_w8a8_variant", _g()[:9] + [7, None]],
                          ["prism_gemm_w4a8_q4k", _k()], [_QG, _qg()]])
    out = subprocess.run([sys.executable, "-c", _CHILD, built, payload], env=env, capture_output=True, text=True,
                         timeout=120)
    assert out.returncode == 0, out.stderr
    res = json.loads(out.stdout.strip().splitlines()[-1])
    if "device_visible" in res:
        pytest.skip("a HIP device is visible despite HIP_VISIBLE_DEVICES=-1: fake-pointer calls not made")
    assert res["status"] == [UNSUP] * 7


def test_library_build_id_matches_sources(built):
    sys.path.insert(0, ROOT)
    from exact_int8_gemm_amd import build, prism
    prism._lib = None
    assert prism.lib().prism_build_id().decode() == build.source_hash()


def test_library_from_other_sources_is_refused(built, monkeypatch):
    """A library whose build id differs from the hash of the sources beside it is not loaded."""
    sys.path.insert(0, ROOT)
    from exact_int8_gemm_amd import build, prism
    monkeypatch.setattr(build, "source_hash", lambda: "f" * 32)
    monkeypatch.setattr(prism, "_lib", None)
    with pytest.raises(RuntimeError, match="built from other sources"):
        prism.lib()
    assert prism._lib is None


def test_build_uses_result_defining_flags():
    sys.path.insert(0, ROOT)
    from exact_int8_gemm_amd import build
    cmd = " ".join(build._compile_cmd("x.hip", "x.o"))
    for flag in ("--offload-arch=gfx950", "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
                 "-fno-gpu-flush-denormals-to-zero", "-packed-fp32-ops"):
        assert flag in cmd, flag


def test_variant_table_matches_header():
    sys.path.insert(0, ROOT)
    from exact_int8_gemm_amd import prism
    d = _defines()
    for name, v in prism.VARIANTS.items():
        assert d["PRISM_VARIANT_" + name.upper().replace("X", "x")] == v, name
    assert d["PRISM_VARIANT_COUNT"] == len(prism.VARIANTS)
