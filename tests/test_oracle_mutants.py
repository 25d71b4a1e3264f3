"""The oracle's pins must catch plausible mistakes.

Each case copies ``oracle/oracle.c``, plants one mistake by a textual edit
(always one that keeps every access in bounds), builds the copy with gcc in a
temporary directory, points the oracle's binding at it and runs the pin
checks of ``test_oracle_pins``: at least one of them must fail.  Everything
here runs on the CPU.
"""
import ctypes
import os
import subprocess

import pytest

import oracle
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, text in oracle.c, replacement, how many occurrences to replace (0 = all))
MUTANTS = [
    ("dropped last k", "for (int64_t k = 0; k < K; ++k)\n                sum += (int64_t)q[m * K + k] * (int64_t)w[n * K + k];",
     "for (int64_t k = 0; k < K - 1; ++k)\n                sum += (int64_t)q[m * K + k] * (int64_t)w[n * K + k];", 1),
    ("reversed k in w", "(int64_t)w[n * K + k]", "(int64_t)w[n * K + (K - 1 - k)]", 1),
    ("wrong sign", "sum += (int64_t)q[m * K + k] * (int64_t)w[n * K + k];",
     "sum -= (int64_t)q[m * K + k] * (int64_t)w[n * K + k];", 1),
    ("nibble order swapped", "(k % 2 == 0) ? (byte & 0x0f) : (byte >> 4)", "(k % 2 == 0) ? (byte >> 4) : (byte & 0x0f)", 1),
    ("nibble unsigned", "nib >= 8 ? nib - 16 : nib", "nib", 1),
    ("round half away from zero", "nearbyintf(t)", "roundf(t)", 1),
    ("clamp to -128", "if (r < -127.0f) r = -127.0f;", "if (r < -128.0f) r = -128.0f;", 1),
    ("reciprocal instead of division", "float t = xr[k] / sc;", "float t = xr[k] * (1.0f / sc);", 1),
    ("scale off by rounding", "float sc = amax / 127.0f;", "float sc = amax * (1.0f / 127.0f);", 1),
    ("non-finite rows not isolated", "if (!isfinite(xr[k])) finite = 0;", "", 1),
    ("epilogue reassociated", "float t = (float)a * s_a[m];\n            y[m * N + n] = t * s_w[n];",
     "float t = s_a[m] * s_w[n];\n            y[m * N + n] = (float)a * t;", 0),
    ("block combine unfused", "f = fmaf((float)p, oracle_f16_to_f32(d[n * NB + b]), f);",
     "{ float pd = (float)p * oracle_f16_to_f32(d[n * NB + b]); f = f + pd; }", 1),
    ("blocks descending", "float f = 0.0f;\n            for (int64_t b = 0; b < NB; ++b) {",
     "float f = 0.0f;\n            for (int64_t b = NB - 1; b >= 0; --b) {", 1),
    ("activation scale applied first", "y[m * N + n] = f * s_a[m];", "y[m * N + n] = f;", 1),
    ("fp16 subnormals off by one", "ldexpf((float)f, -24)", "ldexpf((float)f, -25)", 1),
    ("fp16 bias wrong", "ldexpf((float)(1024 + f), e - 25)", "ldexpf((float)(1024 + f), e - 24)", 1),
    ("static: round half away from zero", "float r = nearbyintf(t); /* half to even; +-inf stays +-inf */",
     "float r = roundf(t);", 1),
    ("static: reciprocal instead of division", "float t = xr[k] / scale;", "float t = xr[k] * (1.0f / scale);", 1),
    ("static: clamp to -128", "/* half to even; +-inf stays +-inf */\n            if (r > 127.0f) r = 127.0f;\n            if (r < -127.0f) r = -127.0f;",
     "/* half to even; +-inf stays +-inf */\n            if (r > 127.0f) r = 127.0f;\n            if (r < -128.0f) r = -128.0f;", 1),
    ("static: NaN rows not isolated", "if (isnan(xr[k])) has_nan = 1;", "", 1),
    ("static: infinities treated as NaN", "if (isnan(xr[k])) has_nan = 1;", "if (!isfinite(xr[k])) has_nan = 1;", 1),
    ("static: scale output inverted", "s[m] = scale;", "s[m] = 1.0f / scale;", 1),
    ("q8_0: big-endian scale", "(uint16_t)(blk[0] | (blk[1] << 8))", "(uint16_t)(blk[1] | (blk[0] << 8))", 1),
    ("q8_0: codes one byte early", "(int8_t)blk[2 + j]", "(int8_t)blk[1 + j]", 1),
    ("q8_0: block stride 33", "(n * NB + b) * 34", "(n * NB + b) * 33", 1),
    ("q8_0: codes reversed", "w[n * K + b * 32 + j] = (int8_t)blk[2 + j];",
     "w[n * K + b * 32 + (31 - j)] = (int8_t)blk[2 + j];", 1),
    ("q4k: high scale bits from the wrong nibble", "*sc = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);",
     "*sc = (s[j + 4] >> 4) | ((s[j - 4] >> 6) << 4);", 1),
    ("q4k: low/high code halves swapped", "return l < 32 ? (qs[32 * g + l] & 15) : (qs[32 * g + l - 32] >> 4);",
     "return l < 32 ? (qs[32 * g + l] >> 4) : (qs[32 * g + l - 32] & 15);", 1),
    ("q4k: codes paired along k", "return l < 32 ? (qs[32 * g + l] & 15) : (qs[32 * g + l - 32] >> 4);",
     "return (i % 2 == 0) ? (qs[i / 2] & 15) : (qs[i / 2] >> 4);", 1),
    ("q4k: min added", "f = fmaf(-(float)sa, Mn, f);", "f = fmaf((float)sa, Mn, f);", 1),
    ("q4k: min term dropped", "f = fmaf(-(float)sa, Mn, f);", "", 1),
    ("q4k: min term before the scale term", "f = fmaf((float)p, D, f);\n                    f = fmaf(-(float)sa, Mn, f);",
     "f = fmaf(-(float)sa, Mn, f);\n                    f = fmaf((float)p, D, f);", 1),
    ("q4k: min term unfused", "f = fmaf(-(float)sa, Mn, f);", "{ float t = -(float)sa * Mn; f = f + t; }", 1),
    ("q4k: d and dmin swapped", "const float d = oracle_f16_to_f32((uint16_t)(sb[0] | (sb[1] << 8)));",
     "const float d = oracle_f16_to_f32((uint16_t)(sb[2] | (sb[3] << 8)));", 0),
    ("q4k repack: header one byte late", "hdr[(n * NS + t) * 16 + i] = sb[i];", "hdr[(n * NS + t) * 16 + i] = sb[(i + 1) % 16];", 1),
    ("q4k repack: codes from the header's end", "w4[n * (K / 2) + t * 128 + i] = sb[16 + i];",
     "w4[n * (K / 2) + t * 128 + i] = sb[12 + i];", 1),
    ("no int32 range check", "if (sum >= INT32_LIMIT || sum < -INT32_LIMIT) {", "if (0) {", 0),
]


def _checks():
    return [
        lambda: pins.test_w8a8_acc_brute_force(3, 5, 7, 1),
        lambda: pins.test_w8a8_acc_brute_force(8, 8, 128, 2),
        lambda: pins.test_w4a8_acc_brute_force(4, 6, 64, 1),
        pins.test_int8_product_table_exhaustive,
        pins.test_int4_decode_exhaustive,
        lambda: pins.test_identity_weights(127),
        pins.test_linearity_symmetry_zero_permutation_split,
        pins.test_extreme_sums_and_int32_bound,
        lambda: pins.test_quantizer_exact_rationals(0),
        pins.test_quantizer_scale_exact_many_magnitudes,
        pins.test_quantizer_properties,
        pins.test_quantizer_special_rows_are_local,
        pins.test_static_quantizer_exact_rationals,
        pins.test_static_quantizer_hand_table,
        pins.test_static_quantizer_equals_dynamic_at_row_absmax,
        pins.test_q8_0_hand_fixture,
        pins.test_q8_0_round_trip_with_struct_packer,
        pins.test_q4_k_hand_fixture,
        pins.test_q4_k_round_trip_with_independent_packer,
        pins.test_q4_k_gemm_within_bound_of_exact_dot_product,
        pins.test_q4_k_gemm_without_mins_is_the_block_scale_gemm,
        lambda: pins.test_q4_k_gemm_exact_rationals(0),
        pins.test_q4_k_fold_order_where_orders_differ,
        pins.test_channel_epilogue_exact_rationals,
        pins.test_w4a8_epilogue_exact_rationals,
        pins.test_f16_to_f32_exhaustive_vs_numpy,
        lambda: pins.test_blockscale_exact_rationals(0),
        pins.test_blockscale_fma_is_fused_not_mul_add,
        pins.test_golden_quantize,
        pins.test_golden_gemms,
    ]


@pytest.mark.parametrize("name,old,new,count", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, monkeypatch, name, old, new, count):
    src = open(SRC).read()
    assert old in src, "mutation site not found: %s" % name
    mutated = src.replace(old, new) if count == 0 else src.replace(old, new, count)
    c = tmp_path / "mutant.c"
    so = tmp_path / "libmutant.so"
    c.write_text(mutated)
    subprocess.run(["gcc", *oracle.CFLAGS, "-o", str(so), str(c), "-lm"], check=True)
    monkeypatch.setattr(oracle, "_lib", oracle.bind(ctypes.CDLL(str(so))))
    failures = 0
    for check in _checks():
        try:
            check()
        except (AssertionError, oracle.OracleError, pytest.fail.Exception):
            failures += 1
    assert failures > 0, "no pin caught the mutant '%s'" % name


def test_unmutated_copy_passes_every_check(tmp_path, monkeypatch):
    so = tmp_path / "libcopy.so"
    subprocess.run(["gcc", *oracle.CFLAGS, "-o", str(so), SRC, "-lm"], check=True)
    monkeypatch.setattr(oracle, "_lib", oracle.bind(ctypes.CDLL(str(so))))
    for check in _checks():
        check()
