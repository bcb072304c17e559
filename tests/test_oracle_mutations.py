"""The pins must catch plausible mistakes in the oracle.

Each mutation plants one mistake in a temporary copy of the oracle's C
source (a flipped sign, a wrong pair index, epsilon outside the root, a
dropped cache length, a transposed page/slot, ...), builds it on the CPU,
points the oracle adapter at it and runs the pin tests: at least one pin
must fail for every mutant.  Nothing here touches a GPU.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_bshd_pins as bshd_pins
from tests import test_oracle_fp8_pins as fp8_pins
from tests import test_oracle_gemv_pins as gemv_pins
from tests import test_oracle_norm_pins as norm_pins
from tests import test_oracle_pins as pins

MUTATIONS = {
    "rotation_sign": ("y[j0] = re * c - im * s;", "y[j0] = re * c + im * s;"),
    "rotation_imag": ("y[j1] = re * s + im * c;", "y[j1] = im * c - re * s;"),
    "cos_sin_swapped": ("double c = (double)row[2 * i];", "double c = (double)row[2 * i + 1];"),
    "half_split_partner": ("uint32_t j1 = start + (interleaved ? 2 * i + 1 : i + R / 2);",
                           "uint32_t j1 = start + (interleaved ? 2 * i + 1 : i + D / 2);"),
    "interleaved_freq_index": ("const float* row = freqs + (uint64_t)pos * R;",
                               "const float* row = freqs + (uint64_t)pos * D;"),
    "position_ignores_cache_len": ("uint64_t pos = (uint64_t)c->cache_lengths[cseq] + (t - off[b]);",
                                   "uint64_t pos = (uint64_t)(t - off[b]);"),
    "position_off_by_one": ("uint64_t pos = (uint64_t)c->cache_lengths[cseq] + (t - off[b]);",
                            "uint64_t pos = (uint64_t)c->cache_lengths[cseq] + (t - off[b]) + (t > 0);"),
    "slot_from_page_index": ("*slot = pos % c->page_size;", "*slot = (pos / c->page_size) % c->page_size;"),
    "v_off_by_one_element": ("const int64_t dst = row_offset(c, w.page, 1, layer_idx, w.slot, h);\n      const int64_t so = c->scales ? scale_offset(c, w.page, 1, layer_idx, w.slot, h) : -1;\n      read_plain(qkv,",
                             "const int64_t dst = row_offset(c, w.page, 1, layer_idx, w.slot, h) + 1;\n      const int64_t so = c->scales ? scale_offset(c, w.page, 1, layer_idx, w.slot, h) : -1;\n      read_plain(qkv,"),
    "layer_ignored": ("(int64_t)layer * c->layer_stride +", ""),
    "eps_outside_root": ("double r = 1.0 / sqrt(ss / (double)D + eps);",
                         "double r = 1.0 / (sqrt(ss / (double)D) + eps);"),
    "norm_sum_not_mean": ("double r = 1.0 / sqrt(ss / (double)D + eps);",
                          "double r = 1.0 / sqrt(ss + eps);"),
    "weight_offset_dropped": ("y[j] = x[j] * r * (g + w);", "y[j] = x[j] * r * g;"),
    "bf16_ties_away": ("double r = nearbyint(x / quantum) * quantum;",
                       "double r = round(x / quantum) * quantum;"),
    "bf16_truncate": ("double r = nearbyint(x / quantum) * quantum;",
                      "double r = trunc(x / quantum) * quantum;"),
    "bf16_no_subnormals": ("if (e < -126) e = -126;", ""),
    "f16_truncate": ("double r = fabs(nearbyint(x / quantum) * quantum);",
                     "double r = fabs(trunc(x / quantum) * quantum);"),
    "f16_no_subnormals": ("if (e < -14) e = -14;", ""),
    "f16_bias": ("ldexp(1.0 + (double)m / 1024.0, e - 15)", "ldexp(1.0 + (double)m / 1024.0, e - 16)"),
    "batch_offset_ignored": ("uint32_t cseq = (uint32_t)b + batch_offset;",
                             "uint32_t cseq = (uint32_t)b;"),
    "radd_adds_twice": ("float sum = cur + add; /* one IEEE binary32 add */",
                        "float sum = cur + add + add;"),
    "radd_halves_swapped": ("(int64_t)(plane * hidden)", "(int64_t)((1 - plane) * hidden)"),
    "unroped_dims_rounded": ("if ((j >= lo && j < hi) || src_dt != dst_dt)", "if (1)"),
    "rope_tail_ignored": ("const uint32_t r0 = rope_tail ? D - R : 0;\n  if (qkv_row_stride",
                          "const uint32_t r0 = 0;\n  if (qkv_row_stride"),
    "e4m3_bias_8": ("v = ldexp(1.0 + (double)m / 8.0, e - 7);", "v = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    "e4m3_truncate": ("double r = isinf(a) ? 448.0 : nearbyint(a / quantum) * quantum;",
                      "double r = isinf(a) ? 448.0 : trunc(a / quantum) * quantum;"),
    "e4m3_no_subnormals": ("if (e < -6) e = -6;", ""),
    "fp8_scale_for_max_240": ("float s = amax / 448.0f;", "float s = amax / 240.0f;"),
    "fp8_dequant_ignores_scale": ("x[j] = (double)((float)orc_e4m3_to_double(codes[j]) * s);",
                                  "x[j] = (double)((float)orc_e4m3_to_double(codes[j]));"),
    "fp8_bf16_scale_not_rounded": ("if (c->scale_dtype == ORC_BF16) s = (float)orc_bf16_to_double(orc_round_bf16((double)s));", ""),
    "fp8_v_scale_in_k_slot": ("const int64_t so = c->scales ? scale_offset(c, w.page, 1, layer_idx, w.slot, h) : -1;\n      read_plain(qkv,",
                              "const int64_t so = c->scales ? scale_offset(c, w.page, 0, layer_idx, w.slot, h) : -1;\n      read_plain(qkv,"),
    "bshd_padded_rows_roped": ("if (s >= valid_lengths[b]) {", "if (s > valid_lengths[b]) {"),
    "bshd_position_ignores_cache_len": ("const uint32_t pos = c->cache_lengths[b] + s;",
                                        "const uint32_t pos = s;"),
    "bshd_k_from_v_plane": ("int64_t dst = row_offset(c, page, 0, layer_idx, slot, h);",
                            "int64_t dst = row_offset(c, page, 1, layer_idx, slot, h);"),
    "gemv_drops_last_k": ("for (uint32_t kk = 0; kk < k; ++kk) {",
                          "for (uint32_t kk = 0; kk + 1 < k; ++kk) {"),
    "gemv_x_row_ignored": ("get(input, dtype, (int64_t)i * (int64_t)input_row_stride + kk)",
                           "get(input, dtype, kk)"),
    "gemv_weight_stride_is_k": ("? (int64_t)j * (int64_t)weight_row_stride + kk",
                                "? (int64_t)j * (int64_t)k + kk"),
    "gemv_transpose_flag_ignored": ("const int64_t widx = transpose_b", "const int64_t widx = 1"),
    "gemv_k_by_n_stride_is_n": (": (int64_t)kk * (int64_t)weight_row_stride + j;",
                                ": (int64_t)kk * (int64_t)n + j;"),
    "gemv_k_by_n_read_as_n_by_k": (": (int64_t)kk * (int64_t)weight_row_stride + j;",
                                   ": (int64_t)j * (int64_t)weight_row_stride + kk;"),
    "partial_norm_eps_outside_root": (
        "r = 1.0 / sqrt(ss / (double)n_normed + (double)epsilon);",
        "r = 1.0 / (sqrt(ss / (double)n_normed) + (double)epsilon);"),
    "partial_norm_mean_over_all_columns": (
        "r = 1.0 / sqrt(ss / (double)n_normed + (double)epsilon);",
        "r = 1.0 / sqrt(ss / (double)n + (double)epsilon);"),
    "partial_norm_sums_all_columns": ("for (uint32_t j = 0; j < n_normed; ++j) ss += y[j] * y[j];",
                                      "for (uint32_t j = 0; j < n; ++j) ss += y[j] * y[j];"),
    "partial_norm_gamma_reversed": ("y[j] * r * get(gamma, dtype, j));",
                                    "y[j] * r * get(gamma, dtype, n_normed - 1 - j));"),
    "partial_norm_uses_weight_offset": ("y[j] * r * get(gamma, dtype, j));",
                                        "y[j] * r * (get(gamma, dtype, j) + weight_offset));"),
    "mbc_false_norm_unrounded": ("double n = round_to(dt, x[j] * r);", "double n = x[j] * r;"),
    "mbc_false_gamma_sum_unrounded": ("double gw = round_to(dt, g + w);", "double gw = g + w;"),
    "mbc_false_product_unrounded": ("y[j] = round_to(dt, n * gw);", "y[j] = n * gw;"),
    "mbc_flag_ignored": ("if (multiply_before_cast) {", "if (1) {"),
    "mbc_flag_inverted": ("if (multiply_before_cast) {", "if (!multiply_before_cast) {"),
    "dual_index_uses_main_eps": (
        "  return orc_qk_rmsnorm_rope_paged(buf, dtype, T, buf_row_stride, index_band, weight_offset,",
        "  orc_band ib_ = *index_band;\n  ib_.epsilon = main_band->epsilon;\n"
        "  return orc_qk_rmsnorm_rope_paged(buf, dtype, T, buf_row_stride, &ib_, weight_offset,"),
    "dual_index_uses_main_cache_lengths": (
        "  return orc_qk_rmsnorm_rope_paged(buf, dtype, T, buf_row_stride, index_band, weight_offset,",
        "  orc_cache ic_ = *index_band->cache;\n  ic_.cache_lengths = main_band->cache->cache_lengths;\n"
        "  orc_band ib_ = *index_band;\n  ib_.cache = &ic_;\n"
        "  return orc_qk_rmsnorm_rope_paged(buf, dtype, T, buf_row_stride, &ib_, weight_offset,"),
    "dual_index_uses_main_gammas": (
        "  return orc_qk_rmsnorm_rope_paged(buf, dtype, T, buf_row_stride, index_band, weight_offset,",
        "  orc_band ib_ = *index_band;\n  ib_.q_gamma = main_band->q_gamma;\n  ib_.k_gamma = main_band->k_gamma;\n"
        "  return orc_qk_rmsnorm_rope_paged(buf, dtype, T, buf_row_stride, &ib_, weight_offset,"),
    "norm_k_rows_in_last_plane": (
        "      const int64_t dst = row_offset(c, w.page, 0, layer_idx, w.slot, h);\n"
        "      const int64_t so = c->scales ? scale_offset(c, w.page, 0, layer_idx, w.slot, h) : -1;\n"
        "      const uint32_t lo",
        "      const int64_t dst = row_offset(c, w.page, c->kv_planes - 1, layer_idx, w.slot, h);\n"
        "      const int64_t so = c->scales ? scale_offset(c, w.page, 0, layer_idx, w.slot, h) : -1;\n"
        "      const uint32_t lo"),
    "unnormed_from_wrong_column": ("          y[j]);\n  }\n  free(y);", "          y[j - n_normed]);\n  }\n  free(y);"),
}

PIN_TESTS = [
    (pins.test_bf16_rounding_golden_cases, {}),
    (pins.test_bf16_rounding_matches_exhaustive_search, {}),
    (pins.test_f16_rounding_golden_cases, {}),
    (pins.test_f16_rounding_matches_numpy, {}),
    (pins.test_tiny_store_matches_complex_brute_force, {"interleaved": True}),
    (pins.test_tiny_store_matches_complex_brute_force, {"interleaved": False}),
    (pins.test_partial_rope_and_ragged_batch_brute_force, {"interleaved": True, "dtype": "bf16"}),
    (pins.test_partial_rope_and_ragged_batch_brute_force, {"interleaved": False, "dtype": "f32"}),
    (pins.test_unit_vectors_give_cos_sin_closed_form, {"interleaved": True}),
    (pins.test_unit_vectors_give_cos_sin_closed_form, {"interleaved": False}),
    (pins.test_roped_dot_product_depends_only_on_position_difference, {}),
    (pins.test_copies_keep_every_bit_including_specials, {}),
    (pins.test_rmsnorm_constant_vector_closed_form, {}),
    (pins.test_rmsnorm_invariants, {}),
    (pins.test_rmsnorm_epsilon_sits_inside_the_root, {}),
    (norm_pins.test_multiply_after_cast_closed_form, {"dtype": "bf16", "interleaved": True}),
    (norm_pins.test_multiply_after_cast_closed_form, {"dtype": "f16", "interleaved": False}),
    (norm_pins.test_multiply_before_cast_true_rounds_once, {"dtype": "bf16"}),
    (norm_pins.test_dual_band_brute_force, {"dtype": "bf16", "interleaved": False}),
    (norm_pins.test_dual_band_brute_force, {"dtype": "f32", "interleaved": True}),
    (pins.test_radd_is_one_binary32_add_per_element, {"dtype": "bf16"}),
    (pins.test_radd_is_one_binary32_add_per_element, {"dtype": "f32"}),
    (pins.test_trailing_partial_rope_brute_force, {"interleaved": False, "dtype": "bf16"}),
    (bshd_pins.test_bshd_matches_complex_brute_force, {"dtype": "bf16", "interleaved": False}),
    (bshd_pins.test_bshd_padded_rows_are_copied_bit_for_bit, {}),
    (fp8_pins.test_e4m3_rounding_golden_cases, {}),
    (fp8_pins.test_e4m3_decode_matches_bit_fields, {}),
    (fp8_pins.test_fp8_store_v_rows_match_binary32_quantization_exactly,
     {"dtype": "bf16", "scale_dtype": "bf16"}),
    (fp8_pins.test_fp8_store_k_rows_are_the_quantized_rotation,
     {"interleaved": True, "scale_dtype": "f32"}),
    (fp8_pins.test_fp8_radd_is_dequantize_add_requantize_bit_for_bit, {}),
    (gemv_pins.test_gemv_matches_exact_rational_sums, {}),
    (gemv_pins.test_partial_norm_closed_form, {}),
    (gemv_pins.test_partial_norm_unit_mean_square_and_scale_invariance, {}),
    (gemv_pins.test_weight_offset_is_not_consumed, {}),
    (gemv_pins.test_rows_are_independent, {}),
    (gemv_pins.test_w_stored_k_by_n_matches_exact_rational_sums, {}),
    (gemv_pins.test_w_stored_k_by_n_is_not_read_as_n_by_k, {}),
]


def _build_mutant(tmp_path, name, old, new):
    src = open(oracle.SRC).read()
    assert src.count(old) >= 1, f"mutation {name}: pattern not found"
    mutated = src.replace(old, new)
    c_path = tmp_path / f"{name}.c"
    c_path.write_text(mutated)
    (tmp_path / "qrp_oracle.h").write_text(open(os.path.join(oracle.HERE, "qrp_oracle.h")).read())
    so = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared", "-w",
                    str(c_path), "-o", str(so), "-lm"], check=True)
    return str(so)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_some_pin_fails_on_mutant(name, tmp_path, monkeypatch):
    old, new = MUTATIONS[name]
    so = _build_mutant(tmp_path, name, old, new)
    monkeypatch.setattr(oracle, "LIB_PATH", so)
    monkeypatch.setattr(oracle, "_lib", None)
    caught = []
    for fn, kwargs in PIN_TESTS:
        try:
            fn(**kwargs)
        except (AssertionError, ValueError, IndexError):
            caught.append(fn.__name__)
            break
    monkeypatch.setattr(oracle, "_lib", None)
    assert caught, f"no pin catches mutation {name}"
