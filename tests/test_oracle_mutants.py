"""Plants plausible mistakes in a copy of the oracle (on the CPU, in a temp
dir) and checks that the pins of test_oracle_pins / test_oracle_codecs catch
every one of them."""

import ctypes
import os
import shutil
import subprocess

import pytest

import oracle
from oracle.build import CFLAGS

from . import test_oracle_absorbed as absorbed
from . import test_oracle_append as append
from . import test_oracle_codecs as codecs
from . import test_oracle_mha as mha
from . import test_oracle_pins as pins
from . import test_oracle_prefill as prefill
from . import test_oracle_ring as ring
from . import test_oracle_rope as rope

HERE = os.path.dirname(os.path.abspath(oracle.__file__))

MUTANTS = {
    "drop_rope_term": ("for (int32_t i = 0; i < dr; ++i) dot += qr[i] * c[dl + i];", ""),
    "scale_over_latent_width": ("1.0 / sqrt((double)(P->d_nope + P->d_rope))",
                                "1.0 / sqrt((double)(P->d_latent + P->d_rope))"),
    "transposed_w_uk": ("const double* wr = Wk + (int64_t)i * dl;\n        for (int32_t j = 0; j < dl; ++j) acc += wr[j] * c[j];\n        k[i] = acc;",
                        "for (int32_t j = 0; j < dl; ++j) acc += Wk[(int64_t)j * dn + i] * c[j];\n        k[i] = acc;"),
    "missing_normalisation": ("for (int32_t i = 0; i < dv; ++i) out_o[i] /= l;", ""),
    "values_from_w_uk": ("Wv[i] = load_elem(P->w_uv, P->w_dtype, (int64_t)h * dv * dl + i);",
                         "Wv[i] = load_elem(P->w_uk, P->w_dtype, (int64_t)h * dv * dl + i);"),
    "last_token_dropped": ("/* pass 2: weighted sum of the rebuilt values W_UV[h]·c_t ([V2] §2.1) */\n    for (int64_t t = 0; t < nt; ++t) {",
                           "/* pass 2 */\n    for (int64_t t = 0; t < nt - 1; ++t) {"),
    "e4m3_bias_8": ("v = ldexp(1.0 + (double)m / 8.0, e - 7);", "v = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    "paged_offset_wrong": ("return page * P->page_size + t % P->page_size;",
                           "return page * P->page_size + (t + 1) % P->page_size;"),
    "lse_base2": ("lse[idx] = m + log(l);", "lse[idx] = m + log2(l);"),
    "combine_ignores_weights": ("out[d] += wgt * up[d];", "out[d] += up[d] / S;"),
    "row_scale_ignored": ("if (P->cache_dtype == ORACLE_E4M3) f = (double)P->row_scale[r];", ""),
    # cache append
    "e4m3_encode_truncates": ("double q = rint(ldexp(a, 3 - k));", "double q = floor(ldexp(a, 3 - k));"),
    "e4m3_encode_subnormal_spacing": ("const double q = rint(ldexp(a, 9));",
                                      "const double q = rint(ldexp(a, 8));"),
    "append_scale_to_240": ("const float s = fmaxf(amax, 0x1p-126f) / 448.0f;",
                            "const float s = fmaxf(amax, 0x1p-126f) / 240.0f;"),
    "append_bf16_truncates": ("if (dhi < dlo || (dhi == dlo && ((lo >> 16) & 1u))) r = hi;", ""),
    "append_row_off_by_one": (": (int64_t)b * seq_stride + slot;", ": (int64_t)b * seq_stride + slot + 1;"),
    "append_ignores_capacity": ("if (t < 0 || (!ring && t >= capacity)) continue;", "if (t < 0) continue;"),
    # ring cache
    "ring_slot_off_by_one": ("const int64_t slot = ring ? t % seq_stride : t;",
                             "const int64_t slot = ring ? (t + 1) % seq_stride : t;"),
    "ring_window_one_short": ("if (P->ring && t0 < L - P->seq_stride) t0 = L - P->seq_stride;",
                              "if (P->ring && t0 < L - P->seq_stride) t0 = L - P->seq_stride + 1;"),
    "ring_decode_row_map": ("if (P->ring) return (int64_t)b * P->seq_stride + t % P->seq_stride;",
                            "if (P->ring) return (int64_t)b * P->seq_stride + (t + 1) % P->seq_stride;"),
    "ring_grow_destination": ("const int64_t rd = (int64_t)b * dst_cap + t % dst_cap;",
                              "const int64_t rd = (int64_t)b * dst_cap + (t + 1) % dst_cap;"),
    # absorb and up-projection
    "absorb_transposed_w_uk": ("out[j] += q * load_elem(w_uk, w_dtype, (h * d_nope + n) * d_latent + j);",
                               "out[j] += q * load_elem(w_uk, w_dtype, (h * d_latent + j) * d_nope + n);"),
    "absorb_drops_rope_copy": ("out[d_latent + j] = load_elem(q_rope, q_dtype, bh * d_rope + j);",
                               "out[d_latent + j] = 0.0;"),
    "absorb_wrong_query_row": ("const double q = load_elem(q_nope, q_dtype, bh * d_nope + n);",
                               "const double q = load_elem(q_nope, q_dtype, h * d_nope + n);"),
    "up_proj_transposed_w_uv": ("acc += load_elem(w_uv, w_dtype, (h * d_v + v) * d_latent + c) * u[bh * d_latent + c];",
                                "acc += load_elem(w_uv, w_dtype, (h * d_latent + c) * d_v + v) * u[bh * d_latent + c];"),
    "up_proj_drops_last_latent": ("for (int32_t c = 0; c < d_latent; ++c)\n        acc += load_elem(w_uv",
                                  "for (int32_t c = 0; c < d_latent - 1; ++c)\n        acc += load_elem(w_uv"),
    "append_unmapped_page_stops": ("if (page < 0) continue; /* no page mapped */",
                                   "if (page < 0) break; /* no page mapped */"),
    # decoupled RoPE
    "rope_sign": ("out[bh * d_r + i] = a * c - b * s;", "out[bh * d_r + i] = a * c + b * s;"),
    "rope_frequency_exponent": ("inv_freq[i] = (float)pow(base, -(2.0 * (double)i) / (double)d_r);",
                                "inv_freq[i] = (float)pow(base, -(1.0 * (double)i) / (double)d_r);"),
    # MHA baseline
    "mha_scale_over_dv": ("const double sc = scale > 0.0 ? scale : 1.0 / sqrt((double)d_qk);",
                          "const double sc = scale > 0.0 ? scale : 1.0 / sqrt((double)d_v);"),
    "mha_missing_normalisation": ("for (int32_t j = 0; j < d_v; ++j) out[j] /= l;", ""),
    "mha_key_stride": ("load_elem(k, dtype, (kv * seq_stride + t) * d_qk + j)",
                       "load_elem(k, dtype, (kv * seq_stride + t) * d_v + j)"),
    "rebuild_key_drops_rope": ("for (int32_t i = 0; i < dr; ++i) kr[dn + i] = c[dl + i];", ""),
    "rebuild_value_uses_w_uk": ("acc += load_elem(P->w_uv, P->w_dtype, ((int64_t)h * dv + i) * dl + j) * c[j];",
                                "acc += load_elem(P->w_uk, P->w_dtype, ((int64_t)h * dv + i) * dl + j) * c[j];"),
    "gqa_strided_groups": ("const int64_t kvh = h / G;", "const int64_t kvh = h % H_kv;"),
    "gqa_values_of_head_zero": ("const int64_t kv = b * H_kv + kvh;", "const int64_t kv = b * H_kv;"),
    "rope_angle_in_double": ("const float theta = pos * inv_freq[i]; /* binary32 product */",
                             "const double theta = (double)pos * (double)inv_freq[i];"),
    # absorbed-form attention and the E4M3 query
    "absorbed_drops_rope": ("for (int32_t j = 0; j < w; ++j) dot += q[j] * c[j];",
                            "for (int32_t j = 0; j < dl; ++j) dot += q[j] * c[j];"),
    "absorbed_query_factor_ignored": ("const double qf = q_dtype == ORACLE_E4M3 ? (double)q_scale[qrow] : 1.0;",
                                      "const double qf = 1.0;"),
    "absorbed_query_factor_transposed": ("const double qf = q_dtype == ORACLE_E4M3 ? (double)q_scale[qrow] : 1.0;",
                                         "const double qf = q_dtype == ORACLE_E4M3 ? (double)q_scale[(int64_t)h * P->B + b] : 1.0;"),
    "absorbed_missing_normalisation": ("    for (int32_t j = 0; j < dl; ++j) out_u[j] /= l;\n    lse[idx] = log(l) + m;\n    if (o)",
                                       "    lse[idx] = log(l) + m;\n    if (o)"),
    "absorbed_transposed_w_uv": ("acc += load_elem(P->w_uv, P->w_dtype, ((int64_t)h * P->d_v + v) * dl + j) * out_u[j];",
                                 "acc += load_elem(P->w_uv, P->w_dtype, ((int64_t)h * dl + j) * P->d_v + v) * out_u[j];"),
    "quantiser_amax_skips_last": ("for (int32_t j = 0; j < w; ++j) amax = fmaxf(amax, fabsf(x[j]));",
                                  "for (int32_t j = 0; j < w - 1; ++j) amax = fmaxf(amax, fabsf(x[j]));"),
}

PIN_CHECKS = [
    lambda: pins.test_matches_library_attention_on_rebuilt_kv((16, 8, 32, 12)),
    lambda: pins.test_matches_library_attention_on_rebuilt_kv((128, 64, 512, 128)),
    pins.test_identity_weights_reduce_to_one_kv_head_attention,
    pins.test_absorbed_form_identity,
    pins.test_single_token_returns_its_value,
    pins.test_zero_query_is_uniform_average,
    pins.test_one_dominant_key_two_level_weights,
    pins.test_common_score_shift,
    lambda: pins.test_split_and_merge_equals_whole((0, 13, 40, 61)),
    pins.test_default_scale_is_one_over_sqrt_nope_plus_rope,
    pins.test_paged_equals_contiguous_and_poison_is_unread,
    pins.test_fp8_rows_are_decoded_codes_times_row_scale,
    codecs.test_e4m3_decode_all_codes,
    append.test_e4m3_encode_returns_every_code_of_its_value,
    append.test_e4m3_encode_ties_go_to_the_even_mantissa,
    lambda: append.test_fp8_append_matches_the_input_quantiser(3.0),
    append.test_bf16_append_rounds_to_nearest_even,
    append.test_append_places_rows_like_the_decode_row_map,
    rope.test_inverse_frequencies,
    rope.test_position_zero_is_the_identity,
    lambda: rope.test_pairs_keep_their_length(2048),
    lambda: rope.test_rotation_angle_is_the_binary32_product(131071),
    rope.test_quarter_turns_of_the_unit_frequency_pair,
    lambda: rope.test_angles_add(100, 28),
    pins.test_absorb_q_and_up_proj_outputs_reproduce_the_naive_decode,
    append.test_unmapped_page_is_skipped,
    lambda: ring.test_ring_decode_is_the_linear_decode_over_the_last_c_tokens(45, 32),
    ring.test_ring_within_capacity_equals_the_linear_cache_bit_for_bit,
    lambda: ring.test_grown_ring_decodes_like_the_window_it_keeps(16, 48, [12, 16, 0]),
    lambda: ring.test_grown_ring_decodes_like_the_window_it_keeps(32, 8, [50, 9, 0]),
    lambda: mha.test_matches_library_attention(192, 128),
    mha.test_mla_is_mha_on_rebuilt_keys_and_values,
    mha.test_closed_forms,
    lambda: mha.test_gqa_matches_library_grouped_attention(8, 2),
    mha.test_mqa_is_mla_with_identity_up_projections,
    prefill.test_rebuilt_keys_and_values_reproduce_the_decode,
    prefill.test_sub_range_is_a_slice_and_paged_equals_contiguous,
    lambda: absorbed.test_absorbed_form_reproduces_the_naive_decode("dsv2_b32_l2k", {}),
    absorbed.test_sub_ranges_and_ring_follow_the_naive_decode,
    absorbed.test_closed_forms,
    absorbed.test_e4m3_query_is_codes_times_its_factor,
    absorbed.test_quantiser_equals_an_independent_one_and_the_cache_rows,
    absorbed.test_absorb_q_fp8_is_the_quantised_absorbed_query,
]


def _build_mutant(tmp, name):
    src = open(os.path.join(HERE, "oracle.c")).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not found in oracle.c"
    d = tmp / name
    d.mkdir()
    (d / "oracle.c").write_text(src.replace(old, new))
    shutil.copy(os.path.join(HERE, "oracle.h"), d / "oracle.h")
    lib = d / "liboracle.so"
    subprocess.run(["gcc", *CFLAGS, "-Wno-unused-variable", "-Wno-unused-but-set-variable",
                    str(d / "oracle.c"), "-o", str(lib), "-lm"], check=True)
    return str(lib)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(tmp_path, name, monkeypatch):
    path = _build_mutant(tmp_path, name)
    good = oracle.lib()
    # a library with the same entry points and signatures, different arithmetic
    mut = ctypes.CDLL(path)
    for fn in ("oracle_mla_decode", "oracle_absorb_q", "oracle_combine", "oracle_up_proj",
               "oracle_decode_bf16", "oracle_decode_e4m3", "oracle_decode_array",
               "oracle_mla_cache_bytes_per_token", "oracle_mha_cache_bytes",
               "oracle_num_threads", "oracle_cache_append", "oracle_encode_e4m3",
               "oracle_rope", "oracle_rope_inv_freq", "oracle_mha_decode", "oracle_ring_grow", "oracle_gqa_decode", "oracle_rebuild_kv",
               "oracle_absorbed_decode", "oracle_quantize_e4m3_rows"):
        getattr(mut, fn).restype = getattr(good, fn).restype
        getattr(mut, fn).argtypes = getattr(good, fn).argtypes
    monkeypatch.setattr(oracle, "_lib", mut)
    caught = 0
    for check in PIN_CHECKS:
        try:
            check()
        except (AssertionError, ValueError):
            caught += 1
    assert caught > 0, f"no pin catches mutant {name}"
