"""The oracle's pins must catch plausible mistakes (CPU only).

Each mutant is a copy of the oracle's C source with one planted mistake (a
dropped term, a wrong sign, a swapped operand or index, a wrong constant),
compiled with gcc into a temporary library.  The pin tests are then re-run
against that library; at least one of them must fail.  Nothing here touches
the HIP path.
"""
import os

import numpy as np
import pytest

import oracle
from tests import test_oracle_attention as TA
from tests import test_oracle_quant as TQ
from tests import test_oracle_prologue as TP

SRC = os.path.join(os.path.dirname(oracle.__file__), "hifa4_oracle.c")

# (name, original text, planted text, occurrence index)
MUTANTS = [
    ("tie_to_odd_code", "c = (i % 2u == 0u) ? i : i + 1;", "c = (i % 2u == 0u) ? i + 1 : i;", 0),
    ("scale_exponent_off_by_one", "e = ex - 1 - 2;", "e = ex - 2;", 0),
    ("negative_zero_loses_sign", "unsigned sign = signbit(y) ? 8u : 0u;",
     "unsigned sign = (y < 0) ? 8u : 0u;", 0),
    ("smooth_direction_swapped", "v = divide ? v / s[j] : v * s[j];",
     "v = divide ? v * s[j] : v / s[j];", 0),
    ("qk_nibble_order_swapped", "(unsigned char)(blk[k] | (blk[k + 1] << 4))",
     "(unsigned char)(blk[k + 1] | (blk[k] << 4))", 0),
    ("v_nibble_order_swapped", "(unsigned char)(blk[k] | (blk[k + 1] << 4))",
     "(unsigned char)(blk[k + 1] | (blk[k] << 4))", 1),
    ("v_block_transposed", "codes[(blkrow * d + c) * 16 + k / 2]",
     "codes[(blkrow * 16 + k / 2) * d + c]", 0),
    ("alpha_sign_flipped", "double alpha = exp(m - m_new);", "double alpha = exp(m_new - m);", 0),
    ("normaliser_from_unquantised_p", "l = alpha * l + sumPh;", "l = alpha * l + sumP;", 0),
    ("numerator_from_unquantised_p", "double p = Ph[u];", "double p = P[u];", 0),
    ("causal_not_bottom_right", "(long)i + L - c->Sq < last) last = (long)i + L - c->Sq;",
     "(long)i < last) last = (long)i;", 0),
    ("gqa_head_map_modulo", "const int g = h / (c->Hq / c->Hkv);", "const int g = h % c->Hkv;", 0),
    ("p_not_quantised", "if (c->quant_p) {", "if (0) {", 0),
    ("rescale_dropped", "for (int j = 0; j < d; j++) acc_c[j] *= alpha;", "", 0),
    ("merge_weight_dropped", "lsum = a_old * lsum + a_new * l;", "lsum = a_old * lsum + l;", 0),
    ("sm_scale_dropped", "s *= c->sm_scale;", "s *= 1.0;", 0),
    ("lse_from_naive_sum", "J->lse[out] = M + log(lsum) -", "J->lse[out] = M + log(lnsum) -", 0),
    ("p_shift_lse_correction_dropped", "J->lse[out] = M + log(lsum) - c->p_shift * M_LN2;",
     "J->lse[out] = M + log(lsum);", 0),
    ("p_shift_sign_flipped", "P[u] = exp(S[u] - m_new + c->p_shift * M_LN2);",
     "P[u] = exp(S[u] - m_new - c->p_shift * M_LN2);", 0),
    ("p_block_misaligned", "for (long a0 = t0 - (t0 % 32); a0 < t1; a0 += 32)",
     "for (long a0 = t0 - (t0 % 32) - 16; a0 < t1; a0 += 32)", 0),
    ("v_tail_amax_over_padding", "col[k] = k < n ? (double)xh[(size_t)(t0 + k) * d + c] : 0.0;",
     "col[k] = (double)xh[(size_t)((t0 + k) % S) * d + c];", 0),
    ("lazy_threshold_ignored", "double m_new = smax > m + c->tau * M_LN2 ? smax : m;",
     "double m_new = smax > m ? smax : m;", 0),
    ("lazy_threshold_in_natural_units", "double m_new = smax > m + c->tau * M_LN2 ? smax : m;",
     "double m_new = smax > m + c->tau ? smax : m;", 0),
    ("split_phase_sign_flipped", "cend = ((c0 + phase) / chunk + 1) * chunk - phase;",
     "cend = ((c0 + phase) / chunk + 1) * chunk + phase;", 0),
    ("split_phase_ignored", "cend = ((c0 + phase) / chunk + 1) * chunk - phase;",
     "cend = (c0 / chunk + 1) * chunk;", 0),
    ("rope_first_half_sign_flipped", "o[j] = ac - bs;", "o[j] = ac + bs;", 0),
    ("rope_second_half_sign_flipped", "o[j + half] = bc + as;", "o[j + half] = bc - as;", 0),
    ("rope_position_offset_ignored", "const long pos = pos0 + r % S;", "const long pos = r % S;", 0),
    ("calibration_over_all_query_heads", "for (int h = g * G; h < (g + 1) * G; h++) {",
     "for (int h = 0; h < Hq; h++) {", 0),
    ("calibration_ratio_inverted", "(float)pow(km / qm, alpha)", "(float)pow(qm / km, alpha)", 0),
    ("noclip_rule_ignored", "if (rule == 1 && amax > ldexp(6.0, e)) e += 1;", "", 0),
    ("noclip_boundary_inclusive", "if (rule == 1 && amax > ldexp(6.0, e)) e += 1;",
     "if (rule == 1 && amax >= ldexp(6.0, e)) e += 1;", 0),
    ("p_rule_not_passed", "(void)oracle_mx_block(blk, 32, 1, codes, dq, 1, c->p_rule);",
     "(void)oracle_mx_block(blk, 32, 1, codes, dq, 1, 0);", 0),
    ("eps_tile_row_index_by_key_tile", "J->n_qt + i / c->br) * J->n_kt",
     "J->n_qt + i / c->bc) * J->n_kt", 0),
    ("eps_rows_without_mass_counted", "if (J->eps_sum && sumP > 0.0) {", "if (J->eps_sum) {", 0),
    ("eps_row_ratio_inverted", "J->eps_sum[ti] += sumPh / sumP - 1.0;",
     "J->eps_sum[ti] += sumP / sumPh - 1.0;", 0),
    ("eps_pooled_ratio_inverted", "pooled[t] = ph_sum[t] / p_sum[t] - 1.0;",
     "pooled[t] = p_sum[t] / ph_sum[t] - 1.0;", 0),
    ("eps_pooled_from_unquantised_p", "J->ph_sum[ti] += sumPh;", "J->ph_sum[ti] += sumP;", 0),
    ("eps_mean_not_divided_by_rows", "mean[t] = eps_sum[t] / eps_cnt[t];",
     "mean[t] = eps_sum[t];", 0),
    ("dot_product_drops_last_channel", "for (int j = 0; j < d; j++) s += qr[j] * kr[j];",
     "for (int j = 0; j < d - 1; j++) s += qr[j] * kr[j];", 0),
]


def _pin_checks():
    """The pin tests, as plain callables (each raises on failure)."""
    checks = [
        TQ.test_e2m1_golden,
        TQ.test_e2m1_sweep_against_brute_force,
        TQ.test_quantize_rows_layout_and_smooth_direction,
        TQ.test_quantize_v_layout_tail_block,
        TQ.test_mx_block_idempotent_and_on_grid_round_trip,
    ]
    for name, x, sc, codes in TQ._golden_blocks():
        checks.append(lambda x=x, sc=sc, codes=codes, name=name: TQ.test_mx_block_golden(name, x, sc, codes))
    for name, x, sc, codes in TQ._golden_blocks("mx_blocks_noclip.txt"):
        checks.append(lambda x=x, sc=sc, codes=codes, name=name:
                      TQ.test_mx_block_noclip_golden(name, x, sc, codes))
    checks.append(TQ.test_mx_block_noclip_is_the_smallest_unsaturated_exponent)
    for case in TA.CASES:
        checks.append(lambda case=case: TA.test_exact_mode_equals_textbook_softmax(case, 64, 0.0))
    checks += [
        lambda: TA.test_single_tile_mxfp4_p_closed_form(75, 0),
        lambda: TA.test_p_shift_closed_form(0.3),
        lambda: TA.test_p_shift_leaves_exact_attention_unchanged(0.37),
        lambda: TA.test_single_tile_mxfp4_p_closed_form(160, 1),
        lambda: TA.test_lazy_rescale_frame_hand_worked(8.0, 64, 1.0),
        lambda: TA.test_lazy_rescale_frame_hand_worked(2.0, 32, 1.7),
        lambda: TA.test_smooth_qk_invariance_exact(True),
        lambda: TA.test_p_reordering_convex_weights(True, 64, 8.0),
        TA.test_inconsistent_normaliser_is_coherent_row_scaling,
        TA.test_epsilon_tiles_hand_worked_two_by_two,
        lambda: TA.test_epsilon_tiles_single_key_tile_closed_form(0),
        lambda: TA.test_split_k_mxfp4_equals_merge_of_chunk_runs(64),
        lambda: TA.test_split_k_exact_equals_unsplit(128),
        lambda: TA.test_split_phase_mxfp4_equals_merge_of_runs(128, [[0, 64], [64, 0]]),
        TP.test_rope_identity_and_quarter_turn_are_exact,
        TP.test_rope_uses_the_tokens_position_row,
        TP.test_rope_preserves_pair_norms_and_inverts,
        TP.test_calibration_hand_worked,
        lambda: TP.test_calibration_balances_the_smoothed_maxima(0.25),
    ]
    return checks


def test_unmutated_oracle_passes_every_check():
    for chk in _pin_checks():
        chk()


@pytest.mark.parametrize("name,orig,planted,occ", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, orig, planted, occ, tmp_path):
    src = open(SRC).read()
    pos = -1
    for _ in range(occ + 1):
        pos = src.index(orig, pos + 1)
    mutated = src[:pos] + planted + src[pos + len(orig):]
    assert mutated != src
    msrc = tmp_path / "mutant.c"
    msrc.write_text(mutated)
    lib = oracle.build(str(msrc), str(tmp_path / "libmutant.so"))
    caught = []
    with oracle.use_library(lib), np.errstate(all="ignore"):
        for chk in _pin_checks():
            try:
                chk()
            except (AssertionError, ValueError, FloatingPointError) as e:  # noqa: PERF203
                caught.append(type(e).__name__)
                break
    assert caught, "planted mistake %r passed every pin" % name
