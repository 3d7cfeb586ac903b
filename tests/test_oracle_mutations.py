"""Mutation checks for the oracle pins.

Each case plants one plausible mistake in the oracle's C++ source (a one-line
textual change to a copy of oracle/*.cpp), builds that copy with the oracle's
own flags into a separate library, runs one pin against it and requires the
pin to fail. This shows that every part of the oracle is constrained by a
pin. The mutants are built once per session, in parallel."""
import concurrent.futures as cf
import os
import shutil
import tempfile

import pytest

import oracle
import tests.test_oracle_pins as pins

SRC = os.path.dirname(os.path.abspath(oracle.__file__))
FILES = ["quant.cpp", "attention.cpp", "sage.cpp", "impl.h", "oracle.h"]

MUTATIONS = [
    # (id, file, old text, new text, pin, pin args)
    # ---- quantization ([QK-MMAC] §2.1, §4)
    ("round_half_up", "quant.cpp", "float c = std::nearbyint(r);", "float c = std::floor(r + 0.5f);",
     pins.test_quant_worked_ties_from_golden, ()),
    ("scale_divisor_128", "quant.cpp", "const float s = amax / 127.0f;", "const float s = amax / 128.0f;",
     pins.test_quant_properties, ()),
    ("scale_reciprocal_multiply", "quant.cpp", "const float r = x[i] / s;", "const float r = x[i] * (1.0f / s);",
     pins.test_quant_near_ties_against_fp64_quotient, ()),
    # ---- the paged cache ([QK-MMAC] §3)
    ("k_scale_wrong_slot", "quant.cpp", "k_scale[bh * kBlock + off] = s;",
     "k_scale[bh * kBlock + (off + 1) % kBlock] = s;", pins.test_cache_layout_elementwise, (False,)),
    ("v_channels_reversed", "quant.cpp", "static_cast<uint16_t*>(v_cache)[(bh * d + i) * kBlock + off] = vr[i];",
     "static_cast<uint16_t*>(v_cache)[(bh * d + i) * kBlock + off] = vr[d - 1 - i];",
     pins.test_cache_layout_elementwise, (False,)),
    ("gather_token_major_chunks", "quant.cpp",
     "kq[(int64_t)t * d + i] = k_cache[((bh * (d / 16) + i / 16) * kBlock + off) * 16 + i % 16];",
     "kq[(int64_t)t * d + i] = k_cache[((bh * kBlock + off) * (d / 16) + i / 16) * 16 + i % 16];",
     pins.test_qk_brute_force_int64, (33,)),
    ("gather_ignores_block_table", "quant.cpp", "const int64_t bh = (int64_t)table_row[t / kBlock] * H + kvh;",
     "const int64_t bh = (int64_t)(t / kBlock) * H + kvh;",
     pins.test_decode_equals_textbook_attention_of_dequantized, (2, 128, True)),
    # ---- scores, softmax, P.V ([QK-MMAC] §1, §5)
    ("dropped_key_scale", "attention.cpp", "* (double)q_scale * (double)g.sk[t] * scale;", "* (double)q_scale * scale;",
     pins.test_decode_equals_textbook_attention_of_dequantized, (6, 64, False)),
    ("dropped_query_scale", "attention.cpp", "* (double)q_scale * (double)g.sk[t] * scale;",
     "* (double)g.sk[t] * scale;", pins.test_decode_equals_textbook_attention_of_dequantized, (6, 64, False)),
    ("gqa_interleaved_heads", "attention.cpp", "const Gathered g = gather(c, s, ctx[s], h / G);",
     "const Gathered g = gather(c, s, ctx[s], h % c->Hkv);",
     pins.test_decode_equals_textbook_attention_of_dequantized, (2, 128, True)),
    ("prefill_gqa_interleaved_heads", "attention.cpp", "const Gathered g = gather(c, s, n, h / G);\n      std::vector<double> sr(n);\n      for",
     "const Gathered g = gather(c, s, n, h % c->Hkv);\n      std::vector<double> sr(n);\n      for",
     pins.test_prefill_equals_textbook_masked_attention, ()),
    ("softmax_sign_slip", "attention.cpp", "const double p = std::exp(s[j] - m);         // masked keys",
     "const double p = std::exp(m - s[j]);         // masked keys",
     pins.test_decode_softmax_rows_sum_to_one_via_one_hot_v, ()),
    ("softmax_unnormalized", "attention.cpp", "  for (int32_t c = 0; c < d; ++c) out[c] /= l;\n  return m;",
     "  return m;", pins.test_decode_softmax_rows_sum_to_one_via_one_hot_v, ()),
    ("decode_drops_last_token", "attention.cpp",
     "softmax_pv(sr.data(), ctx[s], g.v.data(), d, d, out + row * d);",
     "softmax_pv(sr.data(), ctx[s] - 1, g.v.data(), d, d, out + row * d);",
     pins.test_decode_equals_textbook_attention_of_dequantized, (6, 64, False)),
    ("combine_unweighted_denominator", "attention.cpp", "den += w * l[j];", "den += l[j];",
     pins.test_split_equals_unsplit, (8,)),
    ("split_segment_off_by_a_block", "attention.cpp", "bounds[2 * j + 1] = std::min((j + 1) * L, ctx);",
     "bounds[2 * j + 1] = std::min((j + 1) * L - 16, ctx);", pins.test_split_segments_cover_context, ()),
    ("prefill_causal_off_by_one", "attention.cpp", "std::min<int64_t>(pos + 1, n);", "std::min<int64_t>(pos, n);",
     pins.test_prefill_equals_textbook_masked_attention, ()),
    ("prefill_top_left_alignment", "attention.cpp", "const int64_t pos = (int64_t)n - tq + r;",
     "const int64_t pos = r;", pins.test_prefill_equals_textbook_masked_attention, ()),
    # ---- chunked prefill with the FP8 P.V product
    ("prefill_fp8_scale_divisor_256", "attention.cpp", "const float sc = amax / 448.0f;\n    scales[ch] = sc;",
     "const float sc = amax / 256.0f;\n    scales[ch] = sc;",
     pins.test_prefill_fp8_v_codes_are_per_channel_over_the_whole_context, (False,)),
    ("prefill_fp8_scale_skips_last_token", "attention.cpp",
     "for (int32_t t = 0; t < ctx; ++t) amax = std::max(amax, std::fabs(v[(int64_t)t * d + ch]));",
     "for (int32_t t = 0; t < ctx - 1; ++t) amax = std::max(amax, std::fabs(v[(int64_t)t * d + ch]));",
     pins.test_prefill_fp8_a_late_key_sets_the_channel_scale, ()),
    ("prefill_fp8_p_scale_256", "attention.cpp", "e4m3_encode1(448.0 * p[j])", "e4m3_encode1(256.0 * p[j])",
     pins.test_prefill_fp8_first_rows_of_a_fresh_chunk_closed_form, ()),
    ("prefill_fp8_exact_p_in_numerator", "attention.cpp", "o[ch] += p8[j] * vj[ch];",
     "o[ch] += 448.0 * p[j] * vj[ch];", pins.test_prefill_fp8_first_rows_of_a_fresh_chunk_closed_form, ()),
    ("prefill_fp8_output_unscaled", "attention.cpp", "out[row * d + ch] = o[ch] / l8 * (double)svc[ch];",
     "out[row * d + ch] = o[ch] / l8;", pins.test_prefill_fp8_first_rows_of_a_fresh_chunk_closed_form, ()),
    ("prefill_fp8_gqa_interleaved_heads", "attention.cpp", "or_paged_v_fp8(c, s, n, h / G, codes.data(), svc.data());",
     "or_paged_v_fp8(c, s, n, h % c->Hkv, codes.data(), svc.data());",
     pins.test_prefill_fp8_zero_queries_give_the_mean_of_the_visible_rounded_values, ()),
    ("prefill_fp8_sigma_one_rounding", "attention.cpp",
     "const double ee = e56 * e56 + e448 * e448;\n            const double* vj = v8.data()",
     "const double ee = e448 * e448;\n            const double* vj = v8.data()",
     pins.test_prefill_fp8_tolerance_model_is_calibrated_by_random_references, ()),
    # ---- dense SageAttention-style path
    ("dense_key_block_size", "sage.cpp", "* nkb + j / g->k_block]", "* nkb + j / g->q_block]",
     pins.test_dense_equals_textbook_attention_of_dequantized, (False, None)),
    ("dense_causal_top_left", "sage.cpp", "std::min<int64_t>(i + (g->Nk - g->Nq), (int64_t)g->Nk - 1)",
     "std::min<int64_t>(i, (int64_t)g->Nk - 1)", pins.test_dense_equals_textbook_attention_of_dequantized,
     (True, 260)),
    ("dense_wrong_value_head", "sage.cpp", "const double* vb = v + ((int64_t)b * g->Nk * g->Hkv + h / G) * d;",
     "const double* vb = v + ((int64_t)b * g->Nk * g->Hkv + (h / G + 1) % g->Hkv) * d;",
     pins.test_dense_equals_textbook_attention_of_dequantized, (False, None)),
    ("mean_accumulated_in_fp32", "sage.cpp", "        double sum = 0.0;", "        float sum = 0.0f;",
     pins.test_sage_mean_is_exact_sum, ()),
    ("smoothing_sign", "sage.cpp", "x = x - mu[((int64_t)b * g->Hkv + h) * g->d + c];       // fl32(K - mu)",
     "x = x + mu[((int64_t)b * g->Hkv + h) * g->d + c];       // fl32(K - mu)",
     pins.test_sage_per_block_scales_brute_force, ()),
    ("block_scale_from_half_the_rows", "sage.cpp", "const int32_t r0 = j * R, r1 = std::min(r0 + R, N);",
     "const int32_t r0 = j * R, r1 = std::min(r0 + R / 2, N);", pins.test_sage_per_block_scales_brute_force, ()),
    ("mean_over_all_sequences", "sage.cpp", "sum += (double)x[(((int64_t)b * N + t) * H + h) * d + c];",
     "sum += (double)x[(((int64_t)(t % B) * N + t) * H + h) * d + c];",
     pins.test_varlen_equal_lengths_is_the_batched_forward, (False,)),
    ("lse_log2_instead_of_ln", "attention.cpp", "  return m + std::log(l);", "  return m + std::log2(l);",
     pins.test_lse_of_equal_scores_is_log_of_visible_count, (False, None)),
    ("lse_drops_max_shift", "attention.cpp", "  return m + std::log(l);", "  return std::log(l);",
     pins.test_lse_equals_direct_sum_over_scores, ()),
    ("lse_correction_sign", "sage.cpp", "for (size_t i = 0; i < l.size(); ++i) l[i] += corr[i];",
     "for (size_t i = 0; i < l.size(); ++i) l[i] -= corr[i];", pins.test_lse_correction_restores_constant_key_scores,
     ()),
    ("lse_correction_head_of_group", "sage.cpp", "(double)k_mean[((int64_t)b * Hkv + h / G) * d + c];",
     "(double)k_mean[((int64_t)b * Hkv + h % Hkv) * d + c];", pins.test_lse_correction_restores_constant_key_scores,
     ()),
    ("smooth_v_no_add_back", "sage.cpp", "+= (double)mu_v[((int64_t)b * Hkv + h / G) * d + c];",
     "+= 0.0 * (double)mu_v[((int64_t)b * Hkv + h / G) * d + c];", pins.test_smooth_v_adds_the_mean_back, ()),
    ("mean_divisor_n_minus_1", "sage.cpp", "mu[((int64_t)b * H + h) * d + c] = (float)(sum / (double)N);",
     "mu[((int64_t)b * H + h) * d + c] = (float)(sum / (double)(N - 1));", pins.test_smooth_v_adds_the_mean_back,
     ()),
    ("varlen_keys_at_query_offsets", "sage.cpp",
     "k_bits + (int64_t)k0 * Hkv * d, v_bits + (int64_t)k0 * Hkv * d",
     "k_bits + (int64_t)q0 * Hkv * d, v_bits + (int64_t)q0 * Hkv * d",
     pins.test_varlen_equal_lengths_is_the_batched_forward, (False,)),
    ("varlen_lse_rows_reversed", "sage.cpp", "lse[(int64_t)h * total_q + q0 + i] = l[(int64_t)h * (q1 - q0) + i];",
     "lse[(int64_t)h * total_q + q0 + i] = l[(int64_t)h * (q1 - q0) + (q1 - q0 - 1 - i)];",
     pins.test_varlen_equal_lengths_is_the_batched_forward, (True,)),
    # ---- rotary embedding ahead of quantization ([QK-MMAC] §4)
    ("rope_sign", "quant.cpp", "o[ia] = ac - bs;", "o[ia] = ac + bs;", pins.test_rope_pairs_rotate_as_complex_numbers,
     (True,)),
    ("rope_cos_sin_swapped", "quant.cpp", "const float c = cs[i], s = cs[half + i];",
     "const float s = cs[i], c = cs[half + i];", pins.test_rope_position_zero_is_identity, (True,)),
    ("rope_pairs_adjacent_for_neox", "quant.cpp", "const int32_t ia = neox ? i : 2 * i, ib = neox ? i + half : 2 * i + 1;",
     "const int32_t ia = 2 * i, ib = 2 * i + 1;", pins.test_rope_interleaved_is_half_pairing_of_permuted_channels, ()),
    ("rope_drops_pass_through", "quant.cpp", "for (int32_t i = 0; i < d; ++i) o[i] = widen1(xr[i], dtype);",
     "for (int32_t i = 0; i < d; ++i) o[i] = 0.0f;", pins.test_rope_pairs_rotate_as_complex_numbers, (False,)),
    ("rope_frequency_of_pair_reversed", "quant.cpp", "const float c = cs[i], s = cs[half + i];",
     "const float c = cs[half - 1 - i], s = cs[rot - 1 - i];", pins.test_rope_pairs_rotate_as_complex_numbers, (True,)),
    ("rope_positions_off_by_one", "quant.cpp", "const float* cs = cos_sin + pos[t] * rot;",
     "const float* cs = cos_sin + (pos[t] > 0 ? pos[t] - 1 : 0) * rot;",
     pins.test_rope_pairs_rotate_as_complex_numbers, (False,)),
    # ---- storage formats
    ("f16_ties_away", "quant.cpp", "double n_ = std::nearbyint(a / std::ldexp(1.0, E - 10));",
     "double n_ = std::floor(a / std::ldexp(1.0, E - 10) + 0.5);", pins.test_f32_to_f16_bits_matches_numpy_rounding,
     ()),
    ("f16_subnormals_flushed", "quant.cpp", "    if (E == -14) b = (uint16_t)n_;",
     "    if (E == -14) b = (uint16_t)(n_ >= 1024.0 ? n_ : 0.0);", pins.test_f32_to_f16_bits_matches_numpy_rounding,
     ()),
    ("bf16_widened_as_f16_bits", "quant.cpp", "const uint32_t u = (uint32_t)bits << 16;",
     "const uint32_t u = (uint32_t)bits << 13;", pins.test_widen_bf16_and_f16_exact, ()),
    ("fp8_ties_away", "quant.cpp", "if (dlo < dhi || (dlo == dhi && (lo & 1) != 0)) code = lo - 1;",
     "if (dlo < dhi) code = lo - 1;", pins.test_e4m3_landmarks_ties_and_saturation, ()),
    ("fp8_subnormal_step", "quant.cpp", "const double mag = e == 0 ? m / 8.0 * std::ldexp(1.0, -6)",
     "const double mag = e == 0 ? m / 8.0 * std::ldexp(1.0, -7)", pins.test_e4m3_landmarks_ties_and_saturation, ()),
    # ---- FP8 (E4M3) P.V
    ("fp8_p_not_rounded", "sage.cpp", "p8[j] = p[j] > 0.0 ? e4m3_decode1(e4m3_encode1(448.0 * p[j])) : 0.0;",
     "p8[j] = 448.0 * p[j];", pins.test_fp8pv_one_visible_key_and_two_key_closed_form, ()),
    ("fp8_v_scale_dropped", "sage.cpp", "out[orow + c] = o[c] / l8 * (double)svc[c] +", "out[orow + c] = o[c] / l8 +",
     pins.test_fp8pv_constant_values_come_back, ()),
    ("fp8_v_not_rounded", "sage.cpp", "vals[i] = sc > 0.0f ? e4m3_decode1(e4m3_encode1((double)(v[i] / sc))) : 0.0;",
     "vals[i] = sc > 0.0f ? (double)(v[i] / sc) : 0.0;", pins.test_v_fp8_per_channel_codes, ()),
    ("fp8_sum_of_unrounded_p", "sage.cpp", "          l8 += p8[j];", "          l8 += 448.0 * p[j];",
     pins.test_fp8pv_constant_values_come_back, ()),
    ("fp8_lse_log2", "sage.cpp", "if (lse != nullptr) lse[li] = m + std::log(l8 / 448.0);",
     "if (lse != nullptr) lse[li] = m + std::log2(l8 / 448.0);", pins.test_fp8pv_lse_of_equal_scores_is_log_of_visible_count,
     (False,)),
    ("fp8_sigma_drops_one_rounding", "sage.cpp", "const double ee = e56 * e56 + e448 * e448;",
     "const double ee = e56 * e56;", pins.test_fp8pv_tolerance_model_is_calibrated_by_random_references, ()),
    ("fp8_sigma_unit_not_relative", "sage.cpp", "const double e56 = 56.0 * p[j] >= sub ? u * w : sub_err / (56.0 * lp);",
     "const double e56 = 56.0 * p[j] >= sub ? u * w * w : sub_err / (56.0 * lp);",
     pins.test_fp8pv_tolerance_model_is_calibrated_by_random_references, ()),
]


@pytest.fixture(scope="session")
def mutant_libs():
    """Build every mutant (in parallel) into a temporary directory; returns
    {id: path to its library}."""
    root = tempfile.mkdtemp(prefix="oracle_mutants_")

    def build(case):
        mid, fname, old, new = case[:4]
        d = os.path.join(root, mid)
        os.makedirs(d)
        for f in FILES:
            shutil.copy(os.path.join(SRC, f), d)
        path = os.path.join(d, fname)
        src = open(path).read()
        assert src.count(old) == 1, f"{mid}: the anchor must occur exactly once in {fname}"
        open(path, "w").write(src.replace(old, new))
        return mid, oracle.build_library(d, os.path.join(d, "liboracle.so"))

    workers = max(1, min(8, os.cpu_count() or 1))
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        libs = dict(ex.map(build, MUTATIONS))
    yield libs
    shutil.rmtree(root, ignore_errors=True)


def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


@pytest.mark.parametrize("case", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pin_catches_mutation(mutant_libs, case):
    mid, _, _, _, pin, args = case
    with oracle.use_library(mutant_libs[mid]):
        assert _fails(pin, *args), "the planted mistake went unnoticed"


def test_unmutated_pins_pass():
    for _, _, _, _, pin, args in MUTATIONS:
        pin(*args)
