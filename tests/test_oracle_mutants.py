"""Plant plausible mistakes into copies of the CPU oracle and check the pins catch each.

Every mutant is a textual edit of ``oracle/qmm_oracle.c`` compiled with gcc
into a temporary directory; the pin checks then run against it.  A mutant
that passes every pin would mean the pins leave that part of the oracle
unchecked.
"""
import ctypes
import os
import subprocess

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "qmm_oracle.c")

# (id, original text, replacement): each is a mistake one could plausibly make.
MUTANTS = [
    ("round_half_away", "float t = rintf(v[i] / s) + (float)z;", "float t = roundf(v[i] / s) + (float)z;"),
    ("no_zero_in_range", "float lo = 0.0f, hi = 0.0f;", "float lo = v[0], hi = v[0];"),
    ("zero_point_sign", "float neg_lo = -lo;", "float neg_lo = lo;"),
    ("levels_2pow_b", "const float qmax = (float)((1 << bits) - 1);", "const float qmax = (float)(1 << bits);"),
    ("dequant_drops_zero", "float d = (float)((int)q[r * cols + c] - (int)zeros[gi]);",
     "float d = (float)((int)q[r * cols + c]);"),
    ("scale_zero_to_tiny", "if (s == 0.0f) s = 1.0f;", "if (s == 0.0f) s = 1e-8f;"),
    ("clamp_before_zero", "float t = rintf(v[i] / s) + (float)z;",
     "float t = rintf(v[i] / s); if (t < 0.0f) t = 0.0f; t += (float)z;"),
    ("sym_levels", "const float qpos = (float)((1 << (bits - 1)) - 1);",
     "const float qpos = (float)(1 << (bits - 1));"),
    ("sym_no_floor", "if (amax < floor_) amax = floor_;", ""),
    ("sym_round_trunc", "float t = rintf(v[i] / s);", "float t = truncf(v[i] / s);"),
    ("pack_swapped_nibbles", "out[r * bytes + j] = (uint8_t)(lo | (hi << 4));",
     "out[r * bytes + j] = (uint8_t)(hi | (lo << 4));"),
    ("codes_plain_order", "word |= (uint32_t)(e[2 * i + 1] & 0xF) << (16 + 4 * i);",
     "word |= (uint32_t)(e[2 * i + 1] & 0xF) << (8 * i + 4);"),
    ("matmul_transposed", "acc += (double)a[i * k + t] * (double)b[j * k + t];",
     "acc += (double)a[i * k + t] * (double)b[t * n + j % n];"),
    ("matmul_f32_sum", "double acc = 0.0;", "float acc = 0.0f;"),
    ("int8_wrong_operand", "s += (int64_t)qa[i * k + t] * (int64_t)qb[j * k + t];",
     "s += (int64_t)qa[i * k + t] * (int64_t)qb[i * k + t];"),
    ("rescale_missing_b", "y[i * n + j] = (double)acc[i * n + j] * (double)a[i] * (double)b[j];",
     "y[i * n + j] = (double)acc[i * n + j] * (double)a[i];"),
    ("smooth_inverted", "s[j] = num / den;", "s[j] = den / num;"),
    ("smooth_no_floor", "float x = cx[j] < fl ? fl : cx[j];", "float x = cx[j];"),
    ("cw_no_floor", "float w = cw[j] < fl ? fl : cw[j];", "float w = cw[j];"),
    ("sqrt_of_ratio", "num = sqrtf(x);\n            den = sqrtf(w);", "num = sqrtf(x / w);\n            den = 1.0f;"),
    ("powf_alpha_swapped", "den = powf(w, 1.0f - alpha);", "den = powf(w, alpha);"),
    ("smooth_div_instead_of_mul", "out[i * cols + j] = a[i * cols + j] * s[j];",
     "out[i * cols + j] = a[i * cols + j] / s[j];"),
    ("col_absmax_signed", "float v = fabsf(a[i * cols + j]);", "float v = a[i * cols + j];"),
    ("f16_round_half_away", "double r = nearbyint(ldexp(a, 10 - e));", "double r = round(ldexp(a, 10 - e));"),
    ("f16_subnormal_truncated", "double r = nearbyint(a * ldexp(1.0, 24));", "double r = floor(a * ldexp(1.0, 24));"),
    ("f16_saturate_to_inf", "if (a >= 65504.0) return (uint16_t)(sign | 0x7BFFu);",
     "if (a >= 65520.0) return (uint16_t)(sign | 0x7C00u);"),
    ("f16_scale_zero_kept", "if (s16 == 0.0f) s16 = 1.0f;", ""),
    ("codes_from_f32_scale", "if (scale_f16) s = f16_scale(s);", ""),
    ("awq_no_normalization", "const double norm = sqrt(mx * mn);", "const double norm = 1.0;"),
    ("awq_last_minimum", "if (a == 0 || e < err[bi]) {", "if (a == 0 || e <= err[bi]) {"),
    ("awq_input_not_rescaled", "oq_scale_columns_div(x, s, t, k, xs);", "oq_scale_columns_mul(x, s, t, k, xs);"),
    ("awq_magnitude_max", "for (int64_t r = 0; r < t; ++r) acc += fabs((double)x[r * k + j]);",
     "for (int64_t r = 0; r < t; ++r) acc = fmax(acc, fabs((double)x[r * k + j]));"),
    ("awq_alpha_inverted", "p[j] = pow(mag[j], alphas[a]);", "p[j] = pow(mag[j], 1.0 - alphas[a]);"),
    ("awq_f16_input_rounded_bf16", "xs[i] = x_f16 ? oq_f16_bits_to_f32(oq_f32_to_f16_bits(xs[i])) : bf16_round(xs[i]);",
     "xs[i] = bf16_round(xs[i]);"),
    ("codes3_halves_swapped", "const int pos = 3 * (rr / 2) + 16 * (rr % 2);",
     "const int pos = 3 * (rr / 2) + 16 * ((rr + 1) % 2);"),
    ("codes3_last_pair_words_reversed", "w[t] |= (uint32_t)((e[30] >> t) & 1u) << 15;",
     "w[2 - t] |= (uint32_t)((e[30] >> t) & 1u) << 15;"),
    ("sym_zero_point_off_by_one", "zf = half;                       /* R22 */", "zf = half - 1.0f;"),
    ("e4m3_round_half_away", "double r = nearbyint(ldexp(a, 3 - e));", "double r = round(ldexp(a, 3 - e));"),
    ("e4m3_bias_8", "return (uint8_t)(sign | (uint8_t)((e + 7) << 3) | (uint8_t)(r - 8.0));",
     "return (uint8_t)(sign | (uint8_t)((e + 8) << 3) | (uint8_t)(r - 8.0));"),
    ("e4m3_subnormal_truncated", "double r = nearbyint(a * ldexp(1.0, 9));", "double r = floor(a * ldexp(1.0, 9));"),
    ("fp8_max_480", "float s = amax / 448.0f;", "float s = amax / 480.0f;"),
    ("fp8_product_transposed",
     "sacc += (double)oq_e4m3_to_f32(qa[i * k + t]) * (double)oq_e4m3_to_f32(qb[j * k + t]);",
     "sacc += (double)oq_e4m3_to_f32(qa[i * k + t]) * (double)oq_e4m3_to_f32(qb[t * n + j % n]);"),
    ("llm_outliers_in_absmax", "for (int64_t p = 0; p < kept; ++p) xr[i * k + idx[p]] = 0.0f;", ""),
    ("llm_threshold_strict", "if (cx[j] >= tau) {", "if (cx[j] > tau) {"),
    ("llm_outlier_term_dropped", "y[i * n + j] += s;", ""),
    ("llm_w16_unrounded",
     "w16[j * cap + p] = x_bf16 ? bf16_round(w) : oq_f16_bits_to_f32(oq_f32_to_f16_bits(w));",
     "w16[j * cap + p] = w;"),
    ("llm_bf16_truncates", "if (dropped > 0x8000u || (dropped == 0x8000u && (top & 1u))) top += 1u;", ""),
    ("llm_cap_keeps_last", "if (kept < cap) idx[kept++] = (int32_t)j;",
     "idx[kept < cap ? kept++ : cap - 1] = (int32_t)j;"),
    ("llm_outlier_wrong_column", "s += (double)x[i * k + idx[p]] * (double)w16[j * cap + p];",
     "s += (double)x[i * k + p] * (double)w16[j * cap + p];"),
]


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


@pytest.mark.parametrize("mid,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(mid, old, new, source, tmp_path):
    assert source.count(old) >= 1, f"mutation site for {mid} not found"
    mutated = source.replace(old, new)
    c_path = tmp_path / f"{mid}.c"
    so_path = tmp_path / f"{mid}.so"
    c_path.write_text(mutated)
    subprocess.check_call(["gcc", *oracle.GCC_FLAGS, "-o", str(so_path), str(c_path), "-lm"])
    saved = oracle._lib
    try:
        oracle._lib = None
        good_lib = oracle.lib()          # installs argtypes on the real library
        mutant = ctypes.CDLL(str(so_path))
        for fn_name in ["oq_asym_quantize", "oq_asym_dequantize", "oq_sym_quantize", "oq_sym_dequantize",
                        "oq_pack_nibbles", "oq_pack_codes", "oq_matmul_nt_f64", "oq_int8_matmul_nt", "oq_rescale_f64",
                        "oq_col_absmax", "oq_smooth_factors", "oq_scale_columns_mul", "oq_scale_columns_div",
                        "oq_threads", "oq_quantize_format", "oq_pack_codes3", "oq_f32_to_f16_array",
                        "oq_f16_to_f32_array", "oq_e4m3_array", "oq_e4m3_decode_array", "oq_fp8_quantize",
                        "oq_fp8_matmul_nt", "oq_llm_int8", "oq_awq_search", "oq_awq_factors"]:
            f = getattr(mutant, fn_name)
            f.argtypes = getattr(good_lib, fn_name).argtypes
            f.restype = ctypes.c_int
        oracle._lib = mutant
        failures = []
        for check in oracle_pins.ALL_CHECKS:
            try:
                check()
            except Exception as e:   # a failed assert, an oracle error status, a bad index
                failures.append((check.__name__, type(e).__name__))
        assert failures, f"mutant {mid} passed every pin"
    finally:
        oracle._lib = saved


def _w8a16_mutants():
    import numpy as np

    def f32(q):
        return np.ascontiguousarray(q, np.int8).astype(np.float32)

    def b64(b):
        return np.asarray(b, np.float32).reshape(-1).astype(np.float64)

    return [
        ("w8a16_no_scale", lambda x, q, b: oracle.matmul_nt_f64(x, f32(q))),
        ("w8a16_scale_divides", lambda x, q, b: oracle.matmul_nt_f64(x, f32(q)) / b64(b)[None, :]),
        ("w8a16_unsigned_codes",
         lambda x, q, b: oracle.matmul_nt_f64(x, np.ascontiguousarray(q, np.int8).view(np.uint8).astype(np.float32))
         * b64(b)[None, :]),
        ("w8a16_scales_reversed", lambda x, q, b: oracle.matmul_nt_f64(x, f32(q)) * b64(b)[::-1][None, :]),
    ]


@pytest.mark.parametrize("mid,fn", _w8a16_mutants(), ids=[m[0] for m in _w8a16_mutants()])
def test_w8a16_pin_catches_mutant(mid, fn, monkeypatch):
    # the weight-only INT8 product lives in the Python layer of the oracle:
    # replace it by a plausible mistake and check its pin fails
    monkeypatch.setattr(oracle, "w8a16_reference", fn)
    with pytest.raises(Exception):
        oracle_pins.check_w8a16_reference()
