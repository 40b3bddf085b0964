"""Planted mistakes: each pin of the oracle must fail on a copy of the oracle that carries a
plausible mistake in the step it pins.

Every case below edits one or two lines of the oracle's C source (oracle.planted_mistake
compiles the edited copy into a temporary library and swaps it in), runs the pins that are
meant to catch that kind of mistake, and asserts that at least one of them fails.  The
mistakes are the ones the pages' own ambiguities invite ("SageAttention2 Technical Report"
summary, 3.4: the sign and source of Delta S in "Smoothing Q", l from P~ in Algorithm 1, the
static 1/448 scale and the 240 of the FNUZ format in "FP8 Quantization for P~V", the alpha
rescale of "Two-Level Accumulation", the V_m add-back of "Optional Smoothing of V";
"SageAttention Guide": truncating INT8 cast; "SageAttention3" summary, 3.4: the E8M0 rule,
the 32-key P block, the 448 x 6 two-level target; the SageBwd sections: the per-block P scale,
sm_scale in the gradients, the smoothing term of dQ), plus the group map of the per-thread
scales and the E4M3 divisor of the QK knob.
"""
import pytest

import oracle
import test_oracle_formats as fmt
import test_oracle_mx as mx
import test_oracle_pins as pins
import test_oracle_qk_e4m3 as qke
import test_oracle_sagebwd as sbw

F, B = "sage_oracle.c", "sagebwd_oracle.c"


def _formats(test):
    def run():
        fmt.L = oracle.lib()  # the formats module binds the library at setup
        test()
    return run


MUTANTS = {
    "group_map_bit3": (
        [(F, "return 2 * (u >> 5) + ((u >> 2) & 1);", "return 2 * (u >> 5) + ((u >> 3) & 1);")],
        [_formats(fmt.test_k_group_map_matches_accumulator_layout)]),
    "delta_s_sign": (
        [(F, "S[x] = (qk_term(h, r, t) + ds[t]) * sm_scale;", "S[x] = (qk_term(h, r, t) - ds[t]) * sm_scale;")],
        [lambda: pins.test_qk_lossless_construction(200, False)]),
    "delta_s_from_khat": (
        [(F, "for (int c = 0; c < d; c++) s += (double)qm[c] * (double)h->gk[(size_t)t * d + c];",
          "for (int c = 0; c < d; c++) s += (double)qm[c] * (double)h->khat[(size_t)t * d + c] * h->dk_key[t];")],
        [pins.test_delta_s_decomposition_is_row_constant]),
    "l_from_quantized_p": (
        [(F, "      sum += Pt[x];\n", "      sum += quant_p(h, Pt[x]) / h->pscale;\n")],
        [lambda: pins.test_row_sum_uses_unquantized_p(64)]),
    "no_alpha_rescale": (
        [(F, "for (int c = 0; c < d; c++) out[c] = alpha * out[c] + R[c];",
          "for (int c = 0; c < d; c++) out[c] = out[c] + R[c];")],
        [lambda: pins.test_pv_lossless_construction(150, False, False)]),
    "no_v_mean_addback": (
        [(F, "out[c] = o + (double)h->vmean[c];", "out[c] = o;")],
        [lambda: pins.test_pv_lossless_construction(150, False, True)]),
    "p_scale_240": (
        [(F, "return orc_e4m3_decode(orc_e4m3_encode(h->pscale * p));",
          "return orc_e4m3_decode(orc_e4m3_encode(240.0 * p));")],
        [lambda: pins.test_pv_lossless_construction(150, False, False)]),
    "int8_truncation": (
        [(F, "float y = nearbyintf(x / scale);", "float y = truncf(x / scale);")],
        [pins.test_quantizer_invariants_and_means]),
    "qk_e4m3_divisor_127": (
        [(F, "  return a / 448.0f;\n}\nstatic float qk_scale", "  return a / 127.0f;\n}\nstatic float qk_scale")],
        [lambda: qke.test_qk_e4m3_lossless_construction(200, 0)]),
    "mx_p_exponent_per_tile": (
        [(F, "for (int x = b0; x < b1; x++) if (Pt[x] > am) am = Pt[x];",
          "for (int x = 0; x < n; x++) if (Pt[x] > am) am = Pt[x];")],
        [mx.test_mx_p_block_exponent_follows_block_max_not_row_max]),
    "e8m0_floor_rule": (
        [(F, "while (e < 127 && amax > 6.0 * ldexp(1.0, e)) e++;", "while (e < 127 && amax >= 8.0 * ldexp(1.0, e)) e++;")],
        [_formats(fmt.test_e8m0_scale_rule), lambda: mx.test_mx_lossless_construction_equals_textbook(192, 128, 0, False)]),
    "two_level_target_448x6": (
        [(F, "const double s1 = two ? pm / 6.0 : 1.0;", "const double s1 = two ? pm / 2688.0 : 1.0;"),
         (F, "Pt[x] = two ? 6.0 * (Pt[x] / pm) : Pt[x];", "Pt[x] = two ? 2688.0 * (Pt[x] / pm) : Pt[x];")],
        [lambda: mx.test_mx_two_level_p_lossless_on_two_levels(256, 256, 64, False)]),
    "sagebwd_static_p_scale": (
        [(B, "double sp = h->identity ? 1.0 : exp(rm - mn) / 127.0;", "double sp = h->identity ? 1.0 : 1.0 / 127.0;")],
        [sbw.test_forward_p_scale_from_block_row_max]),
    "sagebwd_dk_without_sm_scale": (
        [(B, "dk[(size_t)t * d + c] += sk * h.sq[i] * sm_scale;", "dk[(size_t)t * d + c] += sk * h.sq[i];")],
        [sbw.test_two_equal_score_keys_closed_form]),
    "sagebwd_dq_without_smoothing_term": (
        [(B, "dq[(size_t)r * d + c] += sm_scale * rs[r - r0] * (double)h.kmean[c];",
          "dq[(size_t)r * d + c] += 0.0 * rs[r - r0] * (double)h.kmean[c];")],
        [sbw.test_smoothing_k_term_of_dq_closed_form]),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name):
    edits, checks = MUTANTS[name]
    caught = 0
    with oracle.planted_mistake(*edits):
        for check in checks:
            try:
                check()
            except AssertionError:
                caught += 1
    assert caught, f"no pin caught the planted mistake {name}"


def test_pins_pass_on_the_oracle():
    """The same checks pass on the unmodified oracle (so a failure above is the mistake's)."""
    for name in sorted(MUTANTS):
        for check in MUTANTS[name][1]:
            check()
