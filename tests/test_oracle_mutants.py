"""How sharp the oracle's pins are.  Each case plants one plausible mistake in a function of
the oracle (a dropped term, a flipped sign, a wrong index, a strict comparison where the method
is inclusive), on the CPU only, and checks that at least one of the pins named for it then
fails.  The oracle's files are not touched: the mistaken function is compiled from an edited
copy of its source and patched into the module for the duration of the case."""
import inspect
import textwrap

import pytest

from oracle import alodlm_oracle as orc
from tests import test_oracle_pins as pins


def _mutant(name, old, new):
    src = textwrap.dedent(inspect.getsource(getattr(orc, name)))
    assert src.count(old) == 1, "the planted mistake must name exactly one spot of %s" % name
    ns = dict(orc.__dict__)
    exec(compile(src.replace(old, new), "<mutant of %s>" % name, "exec"), ns)
    return ns[name]


# (oracle function, text replaced, mistaken text, pins that must notice)
MUTANTS = {
    "group_mean_a_over_every_row": (
        "readout_commit_group", "a[unresolved].mean()", "a.mean()", [pins.test_readout_group_halt_state]),
    "group_mean_a_after_forced_progress": (
        "readout_commit_group", "unresolved = ~commit", "unresolved = ~commit & (H > H.min())",
        [pins.test_readout_group_halt_state]),
    "group_halt_not_from_zero": (
        "readout_commit_group", "a = lam.copy()", "a = 0.5 * lam", [pins.test_readout_group_halt_state]),
    "rope_turns_the_other_way": (
        "rope", "x1 * c - x2 * s, x2 * c + x1 * s", "x1 * c + x2 * s, x2 * c - x1 * s",
        [pins.test_rope_identity_norm_and_relative_position, pins.test_all_commit_reduces_to_one_fixed_depth_pass]),
    "rope_frequency_exponent_off_by_two": (
        "rope", "(-(np.arange(half, dtype=F64) * 2.0) / hd)", "(-(np.arange(half, dtype=F64)) / hd)",
        [pins.test_all_commit_reduces_to_one_fixed_depth_pass]),
    "rmsnorm_without_eps": (
        "rms_norm", "keepdims=True) + eps)", "keepdims=True))",
        [pins.test_all_commit_reduces_to_one_fixed_depth_pass]),
    "rmsnorm_by_mean_abs": (
        "rms_norm", "np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)",
        "(np.mean(np.abs(x), axis=-1, keepdims=True) + eps)",
        [pins.test_rmsnorm_of_constant_vector_is_gain, pins.test_all_commit_reduces_to_one_fixed_depth_pass]),
    "attention_without_scale": (
        "attention", "k[kv].T / math.sqrt(hd)", "k[kv].T",
        [pins.test_attention_special_cases, pins.test_all_commit_reduces_to_one_fixed_depth_pass]),
    "gqa_heads_taken_modulo": (
        "attention", "kv = (h * Hkv) // Hq", "kv = h % Hkv",
        [pins.test_attention_special_cases, pins.test_all_commit_reduces_to_one_fixed_depth_pass]),
    "silu_sign": (
        "silu", "(1.0 + np.exp(-x))", "(1.0 + np.exp(x))", [pins.test_silu_values]),
    "swiglu_gate_and_up_swapped": (
        "layer_forward", "silu(gu[:, :F]) * gu[:, F:]", "silu(gu[:, F:]) * gu[:, :F]",
        [pins.test_all_commit_reduces_to_one_fixed_depth_pass]),
    "attention_residual_dropped": (
        "layer_forward", "x = x + matmul_t(a, W[p + \"wo\"])", "x = matmul_t(a, W[p + \"wo\"])",
        [pins.test_all_commit_reduces_to_one_fixed_depth_pass]),
    "q_norm_gain_on_keys": (
        "layer_forward", "rms_norm(k, W[p + \"k_norm\"], eps)", "rms_norm(k, W[p + \"q_norm\"], eps)",
        [pins.test_all_commit_reduces_to_one_fixed_depth_pass]),
    "prefill_not_causal": (
        "prefill_sequence", "pos, causal=True, prec=prec", "pos, causal=False, prec=prec",
        [pins.test_prefill_builds_every_slot_and_is_causal]),
    "core_reads_the_deeper_of_loop_and_available": (
        "context_for", "np.minimum(loop, np.asarray(avail", "np.maximum(loop, np.asarray(avail",
        [pins.test_depth_select_reads_min_of_loop_and_available_depth]),
    "entropy_log_term_sign": (
        "readout", "logp = (z - m) - np.log(S)", "logp = (z - m) + np.log(S)",
        [lambda: pins.test_uniform_readout_entropy_is_log_vocab(512, 6.238325)]),
    "entropy_max_shift_dropped": (
        "readout", "logp = (z - m) - np.log(S)", "logp = z - np.log(S)",
        [lambda: pins.test_two_level_entropy_closed_form(6.0)]),
    "boost_subtracted": (
        "readout", "z[i, boost_tok[i]] += float(boost_val[i])", "z[i, boost_tok[i]] -= float(boost_val[i])",
        [pins.test_committed_tokens_are_planted_tokens_when_boost_dominates]),
    "argmax_of_negated_logits": (
        "readout", "tok = np.argmax(z, axis=1)", "tok = np.argmax(-z, axis=1)",
        [pins.test_readout_brute_force_tiny_vocab]),
    "exit_gate_sign": (
        "exit_gate", "np.exp(-t)", "np.exp(t)", [pins.test_exit_gate_sigmoid]),
    "halting_update_not_cumulative": (
        "denoise_step_sequence", "a[rows] + (1.0 - a[rows]) * lam[rows]", "lam[rows]",
        [lambda: pins.test_halting_closed_form(0.42, 0.5, 2)]),
    "halting_strictly_above": (
        "denoise_step_sequence", "mean_a >= tau_halt", "mean_a > tau_halt",
        [lambda: pins.test_halting_closed_form(0.5, 0.75, 2)]),
    "commit_strictly_below": (
        "denoise_step_sequence", "H[rows] <= tau_ent", "H[rows] < tau_ent",
        [pins.test_entropy_equal_to_threshold_commits]),
    "eq3_reset_skipped": (
        "denoise_step_sequence", "h[fixed] = _f64(W[\"embed\"][tokens[fixed]])", "pass",
        [pins.test_eq3_committed_rows_are_token_embeddings]),
    "forced_commit_takes_highest_entropy": (
        "denoise_step_sequence", "cand[np.argmin(Hc)]", "cand[np.argmax(Hc)]",
        [pins.test_uniform_depth_when_nothing_commits_and_halting_is_off]),
    "forced_commit_loop_recorded_positive": (
        "denoise_step_sequence", "commit_loop[forced] = -s_end", "commit_loop[forced] = s_end",
        [pins.test_uniform_readout_forces_lowest_position]),
    "stop_mean_over_all_rows": (
        "denoise_step_sequence", "float(a[U].mean())", "float(a.mean())",
        [pins.test_halting_mean_is_over_unresolved_rows_only]),
    "extend_reads_the_cache_at_depth_one": (
        "extend_sequence", "context_for(cache, dims, k_max, li, depth, avail)",
        "context_for(cache, dims, k_max, li, 1, avail)",
        [pins.test_extend_equals_prefill_of_the_longer_prefix]),
    "philox_nine_rounds": (
        "philox4x32_10", "for rnd in range(10):", "for rnd in range(9):",
        [pins.test_oracle_philox_known_answers]),
    "philox_products_swapped": (
        "philox4x32_10", "p1 & mask, (p0 >> sh)", "p0 & mask, (p1 >> sh)",
        [pins.test_oracle_philox_known_answers]),
    "gumbel_counter_fields_swapped": (
        "gumbel_noise", "np.full(n, s), np.full(n, step)", "np.full(n, step), np.full(n, s)",
        [pins.test_gumbel_noise_range_and_counter_layout]),
    "gumbel_single_log": (
        "gumbel_noise", "-np.log(-np.log(u))", "-np.log(u)",
        [pins.test_gumbel_noise_range_and_counter_layout, pins.test_gumbel_sample_limits]),
    "block_without_mask_still_loops": (
        "denoise_step_sequence", "if not U.any():", "if False:",
        [pins.test_no_mask_no_loop_and_sampled_steps_advance_the_counter]),
    "bf16_residual_stream_rounded": (
        "layer_forward", "x = x + matmul_t(a, W[p + \"wo\"])", "x = _rnd(x + matmul_t(a, W[p + \"wo\"]), prec)",
        [lambda: pins.test_bf16_rounding_points_match_an_independent_forward(True)]),
    "bf16_attention_output_not_rounded": (
        "layer_forward", "a = _rnd(attention(q, keys, vals, allowed, prec)", "a = (attention(q, keys, vals, allowed, prec)",
        [lambda: pins.test_bf16_rounding_points_match_an_independent_forward(True)]),
    "bf16_probabilities_not_rounded": (
        "attention", "(_rnd(p, prec) @ v[kv])", "(p @ v[kv])",
        [lambda: pins.test_bf16_rounding_points_match_an_independent_forward(True)]),
    "bf16_probabilities_rounded_after_normalising": (
        "attention", "(_rnd(p, prec) @ v[kv]) / p.sum(axis=1, keepdims=True)",
        "_rnd(p / p.sum(axis=1, keepdims=True), prec) @ v[kv]",
        [lambda: pins.test_bf16_rounding_points_match_an_independent_forward(True)]),
    "bf16_swiglu_output_not_rounded": (
        "layer_forward", "matmul_t(_rnd(silu(gu[:, :F]) * gu[:, F:], prec)", "matmul_t((silu(gu[:, :F]) * gu[:, F:])",
        [lambda: pins.test_bf16_rounding_points_match_an_independent_forward(True)]),
    "bf16_readout_rows_not_rounded": (
        "denoise_step_sequence", "readout(_rnd(r[rows], prec), W[\"lm_head\"], bt, bv)",
        "readout(r[rows], W[\"lm_head\"], bt, bv)",
        [lambda: pins.test_bf16_rounding_points_match_an_independent_forward(True)]),
    "bf16_value_rows_not_rounded": (
        "layer_forward", "v = _kv_round(qkv[:, (Hq + Hkv) * hd:]", "v = (lambda t, *_: t)(qkv[:, (Hq + Hkv) * hd:]",
        [lambda: pins.test_bf16_rounding_points_match_an_independent_forward(True)]),
    "eviction_keeps_one_depth_too_many": (
        "evict_depths", "range(1, keep + 1)", "range(1, keep + 2)",
        [pins.test_evict_depths_buffer_counts_match_page]),
}


@pytest.mark.parametrize("case", sorted(MUTANTS))
def test_a_planted_mistake_fails_a_pin(case, monkeypatch):
    name, old, new, guards = MUTANTS[case]
    monkeypatch.setattr(orc, name, _mutant(name, old, new))
    caught = []
    for pin in guards:
        try:
            pin()
        except Exception as e:  # an assertion, or a shape / index error the mistake causes
            caught.append(type(e).__name__)
    assert caught, "no pin noticed the planted mistake %r" % case


def test_pins_pass_on_the_unchanged_oracle():
    """The same pins, without a planted mistake, pass (so the failures above are the mistakes')."""
    for _, _, _, guards in MUTANTS.values():
        for pin in guards:
            pin()
