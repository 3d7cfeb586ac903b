"""Mutation checks for the oracle pins.

Each case plants one plausible mistake in the oracle's source on the CPU (a
one-line textual change to one function, re-executed in that module's
namespace and monkeypatched in) and requires that some pin then fails. This
shows that every part of the oracle is constrained by a pin."""
import inspect
import textwrap

import pytest

import oracle
import oracle.attention as oa
import oracle.quant as oq
import oracle.rope as orope
import oracle.fp8 as ofp8
import tests.test_oracle_pins as pins


def _mutant(module, fname, old, new):
    src = textwrap.dedent(inspect.getsource(getattr(module, fname)))
    assert src.count(old) >= 1, f"mutation anchor {old!r} not found in {fname}"
    ns = dict(module.__dict__)
    exec(compile(src.replace(old, new, 1), f"<mutant {fname}>", "exec"), ns)
    return ns[fname]


def _plant(monkeypatch, module, fname, old, new):
    m = _mutant(module, fname, old, new)
    monkeypatch.setattr(module, fname, m)
    if module is oq and hasattr(oa, fname):
        monkeypatch.setattr(oa, fname, m)
    if module is oq and hasattr(orope, fname):
        monkeypatch.setattr(orope, fname, m)
    if hasattr(oracle, fname):
        monkeypatch.setattr(oracle, fname, m)


def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


MUTATIONS = [
    # (id, module, function, old text, new text, pin, pin args)
    ("round_half_up", oq, "quant_rows", "np.rint(r)", "np.floor(r + 0.5)",
     pins.test_quant_worked_ties_from_golden, ()),
    ("scale_divisor_128", oq, "quant_rows", "np.float32(127.0)", "np.float32(128.0)",
     pins.test_quant_properties, ()),
    ("scale_reciprocal_multiply", oq, "quant_rows", "r = (x / denom)",
     "r = (x * (np.float32(1.0) / denom))", pins.test_quant_near_ties_against_fp64_quotient, ()),
    ("k_scale_wrong_slot", oq, "write_kv_values", 'caches["k_scale"][blk, :, off] = ks',
     'caches["k_scale"][blk, :, (off + 1) % BLOCK] = ks', pins.test_cache_layout_elementwise, (False,)),
    ("v_not_transposed", oq, "write_kv_values", 'caches["v_cache"][blk, :, :, off] = v_sel',
     'caches["v_cache"][blk, :, :, off] = v_sel[:, :, ::-1]', pins.test_cache_layout_elementwise, (False,)),
    ("gather_skips_token_chunk_swap", oq, "gather_kv", ".transpose(0, 2, 1, 3)", "",
     pins.test_qk_brute_force_int64, (33,)),
    ("gather_ignores_block_table", oq, "gather_kv", "blocks = np.asarray(table_row[:nblk], np.int64)",
     "blocks = np.sort(np.asarray(table_row[:nblk], np.int64))",
     pins.test_decode_equals_textbook_attention_of_dequantized, (2, 128, True)),
    ("dropped_key_scale", oa, "_decode_scores", " * sk.astype(np.float64)[None, :]", "",
     pins.test_decode_equals_textbook_attention_of_dequantized, (6, 64, False)),
    ("dropped_query_scale", oa, "_decode_scores", " * q_scale.astype(np.float64)[:, None]", "",
     pins.test_decode_equals_textbook_attention_of_dequantized, (6, 64, False)),
    ("gqa_interleaved_heads", oa, "paged_decode", "range(kvh * G, (kvh + 1) * G)",
     "range(kvh, Hq, num_kv_heads)", pins.test_decode_equals_textbook_attention_of_dequantized, (2, 128, True)),
    ("softmax_sign_slip", oa, "_softmax_pv", "np.exp(s - m)", "np.exp(m - s)",
     pins.test_decode_softmax_rows_sum_to_one_via_one_hot_v, ()),
    ("softmax_unnormalized", oa, "_softmax_pv", "o = (p @ v) / np.where(l > 0, l, 1.0)", "o = p @ v",
     pins.test_decode_softmax_rows_sum_to_one_via_one_hot_v, ()),
    ("combine_unweighted_denominator", oa, "paged_decode_split", "den = sum(wj * lj", "den = sum(0 * wj + lj",
     pins.test_split_equals_unsplit, (8,)),
    ("decode_drops_last_token", oa, "paged_decode", "kq, sk, v = gather_kv(caches, block_tables[s], ctx, kvh, v_dtype)",
     "kq, sk, v = gather_kv(caches, block_tables[s], ctx - 1, kvh, v_dtype)",
     pins.test_decode_equals_textbook_attention_of_dequantized, (6, 64, False)),
    ("prefill_causal_off_by_one", oa, "chunked_prefill", "<= pos[:, None]", "< pos[:, None]",
     pins.test_prefill_equals_textbook_masked_attention, ()),
    ("prefill_top_left_alignment", oa, "chunked_prefill", "pos = ctx - tq + (sel - a)", "pos = (sel - a)",
     pins.test_prefill_equals_textbook_masked_attention, ()),
    ("dense_key_block_size", oa, "dense_sage_attention", "kblk = np.arange(Nk) // k_block",
     "kblk = np.arange(Nk) // q_block", pins.test_dense_equals_textbook_attention_of_dequantized, (False, None)),
    ("dense_causal_top_left", oa, "dense_sage_attention", "(qr[:, None] + (Nk - Nq))", "(qr[:, None])",
     pins.test_dense_equals_textbook_attention_of_dequantized, (True, 260)),
    ("dense_transposed_value_head", oa, "dense_sage_attention", "_softmax_pv(s_, v[b, :, kvh])",
     "_softmax_pv(s_, v[b, :, (kvh + 1) % Hkv])", pins.test_dense_equals_textbook_attention_of_dequantized, (False, None)),
    ("mean_accumulated_in_fp32", oq, "sage_quantize", "k.astype(np.float64).sum(axis=1)",
     "k.sum(axis=1, dtype=np.float32).astype(np.float64)", pins.test_sage_mean_is_exact_sum, ()),
    ("smoothing_sign", oq, "sage_quantize", "ks = (k - mu[:, None, :, :])", "ks = (k + mu[:, None, :, :])",
     pins.test_sage_per_block_scales_brute_force, ()),
    ("q_block_rows_64", oq, "sage_quantize", "q_i8, q_scale = per_block(q, q_block)",
     "q_i8, q_scale = per_block(q, 64)", pins.test_sage_per_block_scales_brute_force, ()),
    ("lse_log2_instead_of_ln", oa, "_logsumexp_rows", "mm + np.log(", "mm + np.log2(",
     pins.test_lse_of_equal_scores_is_log_of_visible_count, (False, None)),
    ("lse_drops_max_shift", oa, "_logsumexp_rows", "return np.where(live, mm + np.log(", "return np.where(live, np.log(",
     pins.test_lse_equals_direct_sum_over_scores, ()),
    ("lse_correction_sign", oa, "sage_forward", "lse = lse + sage_lse_correction(", "lse = lse - sage_lse_correction(",
     pins.test_lse_correction_restores_constant_key_scores, ()),
    ("lse_correction_head_of_group", oa, "sage_lse_correction", "np.repeat(np.asarray(k_mean, np.float64), G, axis=1)",
     "np.tile(np.asarray(k_mean, np.float64), (1, G, 1))", pins.test_lse_correction_restores_constant_key_scores, ()),
    ("smooth_v_no_add_back", oa, "sage_forward", "out = out + np.where(live", "out = out + 0 * np.where(live",
     pins.test_smooth_v_adds_the_mean_back, ()),
    ("smooth_v_mean_divisor", oa, "sage_smooth_v", "/ np.float64(N))", "/ np.float64(N - 1))",
     pins.test_smooth_v_adds_the_mean_back, ()),
    ("varlen_keys_at_query_offsets", oa, "sage_varlen_forward", "k[None, k0:k1], v[None, k0:k1]",
     "k[None, q0:q0 + (k1 - k0)], v[None, q0:q0 + (k1 - k0)]", pins.test_varlen_equal_lengths_is_the_batched_forward,
     (False,)),
    ("varlen_lse_rows_by_key_offset", oa, "sage_varlen_forward", "lse[:, q0:q1] = l[0]",
     "lse[:, q0:q1] = l[0][:, ::-1]", pins.test_varlen_equal_lengths_is_the_batched_forward, (True,)),
    ("mean_over_all_sequences", oq, "sage_quantize", "total = k.astype(np.float64).sum(axis=1)",
     "total = k.astype(np.float64).sum(axis=1).mean(axis=0, keepdims=True) + 0 * k[:, 0]",
     pins.test_varlen_equal_lengths_is_the_batched_forward, (False,)),
    ("rope_sign", orope, "apply_rope", "- (b * s).astype(np.float32)", "+ (b * s).astype(np.float32)",
     pins.test_rope_pairs_rotate_as_complex_numbers, (True,)),
    ("rope_cos_sin_swapped", orope, "apply_rope", "c, s = cs[:, None, :half], cs[:, None, half:rot_dim]",
     "s, c = cs[:, None, :half], cs[:, None, half:rot_dim]", pins.test_rope_position_zero_is_identity, (True,)),
    ("rope_pairs_adjacent_for_neox", orope, "_pairs", "return np.arange(half), np.arange(half, rot_dim)",
     "return np.arange(0, rot_dim, 2), np.arange(1, rot_dim, 2)", pins.test_rope_interleaved_is_half_pairing_of_permuted_channels,
     ()),
    ("rope_drops_pass_through", orope, "apply_rope", "out = x.copy()", "out = np.zeros_like(x)",
     pins.test_rope_pairs_rotate_as_complex_numbers, (False,)),
    ("rope_frequency_of_pair_reversed", orope, "apply_rope", "c, s = cs[:, None, :half], cs[:, None, half:rot_dim]",
     "c, s = cs[:, None, :half][..., ::-1], cs[:, None, half:rot_dim][..., ::-1]",
     pins.test_rope_pairs_rotate_as_complex_numbers, (True,)),
    ("rope_positions_off_by_one", orope, "apply_rope", "[np.asarray(positions, np.int64)]",
     "[np.maximum(np.asarray(positions, np.int64) - 1, 0)]", pins.test_rope_pairs_rotate_as_complex_numbers, (False,)),
    ("rope_cache_unrotated", orope, "rope_write_kv_cache", "k_rot = apply_rope(k_bits, dtype, positions, cos_sin, rot_dim, neox)",
     "k_rot = widen(k_bits, dtype)", pins.test_rope_cache_write_holds_rotated_keys, ()),
    ("fp8_no_rescale_of_o", ofp8, "dense_sage_attention_fp8pv", "o = o * alpha[:, None] + p8 @", "o = o + p8 @",
     pins.test_fp8pv_is_within_fp8_error_of_the_16bit_path, ()),
    ("fp8_v_scale_dropped", ofp8, "dense_sage_attention_fp8pv", "* sv[b, kvh].astype(np.float64)", "* 1.0",
     pins.test_fp8pv_constant_values_come_back, ()),
    ("fp8_p_not_rounded", ofp8, "dense_sage_attention_fp8pv", "e4m3_round(top * np.exp(", "(top * np.exp(",
     pins.test_fp8pv_one_visible_key_and_two_key_closed_form, ()),
    ("fp8_v_not_rounded", ofp8, "v_fp8_per_channel", "vals = np.where(live[:, None], e4m3_round(r), 0.0)",
     "vals = np.where(live[:, None], r, 0.0)", pins.test_v_fp8_per_channel_codes, ()),
    ("fp8_slack_in_natural_units", ofp8, "dense_sage_attention_fp8pv", "move = mt > m + slack * np.log(2.0)",
     "move = mt > m + slack * 8", pins.test_fp8pv_slack_changes_only_the_rounding, ()),
    ("fp8_ties_away", ofp8, "e4m3_encode", "((dhi == dlo) & (_POS_CODES[hi] % 2 == 0))", "(dhi == dlo)",
     pins.test_e4m3_landmarks_ties_and_saturation, ()),
]


@pytest.mark.parametrize("case", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pin_catches_mutation(monkeypatch, case):
    _, module, fname, old, new, pin, args = case
    _plant(monkeypatch, module, fname, old, new)
    assert _fails(pin, *args), "the planted mistake went unnoticed"


def test_unmutated_pins_pass():
    for _, _, _, _, _, pin, args in MUTATIONS:
        pin(*args)
