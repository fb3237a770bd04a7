"""Planted mistakes in a copy of the oracle must each fail at least one pin.

Every mutant is a one-line textual edit of ``oracle/oracle.c`` compiled into a
temporary library; the pins of ``pins.py`` run against it on the CPU.  This
shows the pins are strong enough to catch a dropped term, a wrong sign or
index, or a swapped operand anywhere in the oracle.
"""
import os

import pytest

import oracle
from pins import ALL_CHECKS

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "window_off_by_one": ("j < p - (int64_t)window_left", "j <= p - (int64_t)window_left"),
    "window_zero_is_disabled": ("window_left >= 0 && j < p", "window_left > 0 && j < p"),
    "causal_bound_loose": ("if (causal && j > p)", "if (causal && j > p + 1)"),
    "top_left_alignment": ("const int64_t p = (kv_len - qo_len) + (t - qo_indptr[b]);",
                           "const int64_t p = (t - qo_indptr[b]);"),
    "gqa_modulo_map": ("const int32_t hk = h / group;", "const int32_t hk = h % num_kv_heads;"),
    "scale_dropped": ("s[j] = sm_scale * dot;", "s[j] = dot;"),
    "lse_base2": ("lse[out_row * num_qo_heads + h] = m + log(l);",
                  "lse[out_row * num_qo_heads + h] = m + log2(l);"),
    "max_not_subtracted": ("const double w = exp(s[j] - m);", "const double w = exp(s[j]);"),
    "slot_index": ("int64_t slot = j % page_size;", "int64_t slot = (j + 1) % page_size;"),
    "page_index": ("kv_indices[(int64_t)kv_indptr[b] + j / page_size]",
                   "kv_indices[(int64_t)kv_indptr[b] + j / page_size / 2]"),
    "last_page_ignored": ("return (npages - 1) * (int64_t)page_size + kv_last_page_len[b];",
                          "return npages * (int64_t)page_size;"),
    "values_from_keys": ("acc[d] += w * (v_scale * load_elem(v_cache, kv_dtype, voff + d));",
                         "acc[d] += w * (v_scale * load_elem(k_cache, kv_dtype, voff + d));"),
    "empty_lse_zero": ("lse[out_row * num_qo_heads + h] = -INFINITY;",
                       "lse[out_row * num_qo_heads + h] = 0.0;"),
    "merge_weight_sign": ("const double wa = exp(a - s), wb = exp(b - s);",
                          "const double wa = exp(s - a), wb = exp(b - s);"),
    "merge_shift_dropped": ("const double s = M + log(exp(a - M) + exp(b - M));",
                            "const double s = log(exp(a - M) + exp(b - M));"),
    "merge_empty_nonzero": ("s_out[i] = -INFINITY;", "s_out[i] = 0.0;"),
    "half_exponent_bias": ("v = ldexp((double)(1024 + f), e - 25);",
                           "v = ldexp((double)(1024 + f), e - 24);"),
    "half_subnormal_scale": ("v = ldexp((double)f, -24);", "v = ldexp((double)f, -25);"),
    "k_scale_dropped": ("(k_scale * load_elem(k_cache, kv_dtype, koff + d))",
                        "(load_elem(k_cache, kv_dtype, koff + d))"),
    "v_scale_on_keys": ("(k_scale * load_elem(k_cache, kv_dtype, koff + d))",
                        "(v_scale * load_elem(k_cache, kv_dtype, koff + d))"),
    "fp8_bias": ("const int e4 = dtype == ORACLE_FP8_E4M3;\n        const int mbits = e4 ? 3 : 2, bias = e4 ? 7 : 15;",
                 "const int e4 = dtype == ORACLE_FP8_E4M3;\n        const int mbits = e4 ? 3 : 2, bias = e4 ? 8 : 15;"),
    "fp8_encode_bias": ("static uint8_t round_to_fp8(double v, int e4)\n{\n    const int mbits = e4 ? 3 : 2, bias = e4 ? 7 : 15;",
                        "static uint8_t round_to_fp8(double v, int e4)\n{\n    const int mbits = e4 ? 3 : 2, bias = e4 ? 8 : 15;"),
    "fp8_subnormal_scale": ("v = ldexp((double)f, 1 - bias - mbits);",
                            "v = ldexp((double)f, -bias - mbits);"),
    "fp8_ties_away": ("if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0))\n        r += 1.0;\n    return r * q;",
                      "if (frac >= 0.5)\n        r += 1.0;\n    return r * q;"),
    "fp8_overflow_saturates": ("return (uint8_t)(sign | (e4 ? 0x7f : 0x7c));",
                               "return (uint8_t)(sign | (e4 ? 0x7e : 0x7b));"),
    "quantize_multiplies": ("const float y = (float)x / scale;", "const float y = (float)x * scale;"),
    "quantize_skips_16_bit_rounding": (
        "return round_to_fp8(round_to_16((double)y, in_dtype), kv_dtype == ORACLE_FP8_E4M3);",
        "return round_to_fp8((double)y, kv_dtype == ORACLE_FP8_E4M3);"),
    "cap_of_unscaled_logit": ("s[j] = soft_cap * tanh(s[j] / soft_cap);",
                              "s[j] = soft_cap * tanh(dot / soft_cap);"),
    "cap_factor_dropped": ("s[j] = soft_cap * tanh(s[j] / soft_cap);",
                           "s[j] = tanh(s[j] / soft_cap);"),
    "append_values_from_keys": ("memcpy(v_cache + s * row_bytes, v_new + i * row_bytes",
                                "memcpy(v_cache + s * row_bytes, k_new + i * row_bytes"),
    "append_ignores_loc": ("memcpy(k_cache + s * row_bytes, k_new + i * row_bytes",
                           "memcpy(k_cache + i * row_bytes, k_new + i * row_bytes"),
    "append_quant_scale_swapped": (
        "oracle_quantize(in_dtype, load_elem(k_new, in_dtype, i * elems + e), k_scale,",
        "oracle_quantize(in_dtype, load_elem(k_new, in_dtype, i * elems + e), v_scale,"),
    "append_quant_row_offset": ("k_cache[s * elems + e] =", "k_cache[(s ^ 1) * elems + e] ="),
    "indices_start_ignored": ("const int64_t s0 = start ? start[b] : 0;", "const int64_t s0 = 0;"),
    "indptr_not_cumulative": ("kv_indptr[b + 1] = (int32_t)(kv_indptr[b] + n);",
                              "kv_indptr[b + 1] = (int32_t)n;"),
    "indices_map_transposed": ("kv_indices[dst] = map[(int64_t)slot[b] * map_cols + col];",
                               "kv_indices[dst] = map[col * map_rows + slot[b]];"),
    "indices_bad_source_kept": ("kv_indices[dst] = -1;", "kv_indices[dst] = 0;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation target not found once: {old!r}"
    mpath = tmp_path / "oracle_mutant.c"
    mpath.write_text(src.replace(old, new))
    impl = oracle.OracleLib(oracle.compile_source(str(mpath), str(tmp_path / "libmut.so")))
    failed = []
    for check in ALL_CHECKS:
        try:
            check(impl)
        except AssertionError:
            failed.append(check.__name__)
        except ValueError:
            failed.append(check.__name__ + "(error)")
    assert failed, f"no pin caught mutant {name}"
