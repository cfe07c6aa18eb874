"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a temporary copy of the oracle's C source
(a dropped term, a wrong sign or index, a transposed operand, a wrong tie
rule), builds it with gcc, and runs the pins of ``test_oracle_pins`` against
it: at least one pin has to fail.  Runs on the CPU only.
"""
import importlib.util
import os
import subprocess

import pytest

from tests import test_oracle_pins as pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "sla2_oracle.c")

MUTANTS = {
    "combine_weight": ("(1.0 - a) * ol[e]", "a * ol[e]"),
    "linear_over_selected": ("if (hit[j]) continue;", "if (!hit[j]) continue;"),
    "phi_without_plus_one": ("x > 0.0 ? x + 1.0 : exp(x)", "x > 0.0 ? x : exp(x)"),
    "no_softmax_scale": ("double inv = 1.0 / sqrt((double)d);\n    for (int e = 0; e < d; ++e) os[e] = 0.0;\n    if (k == 0) return;\n    long nu",
                         "double inv = 1.0;\n    for (int e = 0; e < d; ++e) os[e] = 0.0;\n    if (k == 0) return;\n    long nu"),
    "projection_transposed": ("(double)W[(size_t)c * d + e]", "(double)W[(size_t)e * d + c]"),
    "pool_divides_by_block_size": ("out[c] /= (double)n;", "out[c] /= (double)bs;"),
    "ties_to_higher_index": ("return x->j - y->j;", "return y->j - x->j;"),
    "sparse_not_normalised": ("    for (int e = 0; e < d; ++e) os[e] /= l;\n    (void)i;", "    (void)i;"),
    "k_rounds_down": ("ceil((double)p->topk_frac", "floor((double)p->topk_frac"),
    "e4m3_ties_to_odd": ("fmod(r, 2.0) != 0.0", "fmod(r, 2.0) == 0.0"),
    "lowbit_no_rescale": ("double resc = (m == -INFINITY) ? 0.0 : exp(m - mn);",
                          "double resc = (m == -INFINITY) ? 0.0 : 1.0;"),
    "no_k_smoothing": ("o->mu[c] = (float)(s / (double)N);", "o->mu[c] = 0.0f;"),
    "p_against_tile_max": ("double pt = exp(lbuf[u - t0] - mn);", "double pt = exp(lbuf[u - t0] - mt);"),
    "p_not_scaled_by_256": ("float f = (float)(256.0 * pt);\n                ph = (double)orc_e4m3_decode(orc_e4m3_encode(f)) / 256.0;",
                            "float f = (float)(pt);\n                ph = (double)orc_e4m3_decode(orc_e4m3_encode(f));"),
    "flip_bound_ignores_rescale": ("double wgt = amb[a].step / 256.0 * exp(amb[a].m - m) / l;",
                                   "double wgt = amb[a].step / 256.0 * exp(m - amb[a].m) / l * 0.25;"),
    "flip_bound_window_narrow": ("double win = abuf[u - t0] + mA +", "double win = abuf[u - t0] +"),
    "denominator_without_phi_q": ("den += pq[c] * Zi[c];", "den += Zi[c];"),
    "alpha_of_wrong_head": ("F->alpha[h]);", "F->alpha[0]);"),
    "alpha_block_ignored": ("F->alpha[(size_t)h * Tq + i]", "F->alpha[(size_t)h * Tq]"),
    "v_scale_wrong_channel": ("(double)F->qt->sv[e]", "(double)F->qt->sv[0]"),
    "v_codes_unused": ("if (p->lowbit_v && F->quantize)", "if (p->lowbit_v && !F->quantize)"),
    "v_scale_not_max": ("            if (v > amax) amax = v;", "            amax = v;"),
    "i8_scale_uses_e4m3_max": ("p->int8_qk ? 127.0f : 448.0f", "p->int8_qk ? 448.0f : 448.0f"),
    "i8_ties_away_from_zero": ("(frac == 0.5 && ((long long)r & 1) != 0)", "(frac == 0.5 && r >= 0.0)"),
    "i8_no_clamp": ("    if (r > 127.0) r = 127.0;\n", ""),
    "i8_codes_unsigned": ("a = (double)(int8_t)Qt->qh[(size_t)t * d + c];", "a = (double)Qt->qh[(size_t)t * d + c];"),
    "i8_k_not_smoothed": ("o->kh[(size_t)t * d + c] = p->int8_qk ? (uint8_t)orc_i8_encode(ks / s)",
                          "o->kh[(size_t)t * d + c] = p->int8_qk ? (uint8_t)orc_i8_encode((ks + o->mu[c]) / s)"),
    "v1_negligible_kept_in_linear": ("    if (v1)\n        for (int r = 0; r < kl; ++r) hit[", "    if (0)\n        for (int r = 0; r < kl; ++r) hit["),
    "v1_proj_transposed": ("(double)Wp[(size_t)c * d + e]", "(double)Wp[(size_t)e * d + c]"),
    "v1_negligible_cut_off_by_one": ("for (int r = Tkv - kl; r < Tkv; ++r)\n            if (mrow)", "for (int r = Tkv - kl - 1; r < Tkv - 1; ++r)\n            if (mrow)"),
    "v1_low_not_clamped": ("    if (k > tkv - kh) k = tkv - kh;\n", ""),
    "v1_sparse_halved": ("o[e] = os[e] + pr;", "o[e] = 0.5 * os[e] + pr;"),
    "phi_softmax_not_normalised": ("    for (int c = 0; c < d; ++c) out[c] /= s;\n", ""),
    "phi_softmax_no_exp": ("        out[c] = exp(out[c] - m);\n", "        out[c] = out[c] - m + 30.0;\n"),
    "soft_topk_tau_multiplies": ("f += sigmoid(x[j] / tau + mid);", "f += sigmoid(x[j] * tau + mid);"),
    "soft_topk_bisection_flipped": ("if (f > 0.0) hi = mid;", "if (f < 0.0) hi = mid;"),
    "soft_topk_grad_no_lambda_term": ("sj / tau * ((double)g[j] - c)", "sj / tau * ((double)g[j])"),
    "route_grad_dk_from_kt": ("dk[(size_t)j * d + e] += gij * qt[(size_t)i * d + e];", "dk[(size_t)j * d + e] += gij * kt[(size_t)j * d + e];"),
    "route_grad_dq_transposed": ("a += qb[(size_t)i * d + c] * dq[(size_t)i * d + e];", "a += qb[(size_t)i * d + e] * dq[(size_t)i * d + c];"),
    "bwd_no_D_term": ("double dl = lw[nu] * (dp - D);", "double dl = lw[nu] * dp;"),
    "bwd_dh_over_selected": ("            if (hit[(size_t)i * Tkv + j]) continue;", "            if (!hit[(size_t)i * Tkv + j]) continue;"),
    "bwd_no_ds": ("                    dsv -= (1.0 - a) * g[e] * olin[e] / den;\n", ""),
    "bwd_elu_prime_one": ("dx[c] = dph[c] * (x > 0.0 ? 1.0 : exp(x));", "dx[c] = dph[c];"),
    "bwd_alpha_sign": ("da += g[e] * (os[e] - olin[e]);", "da += g[e] * (olin[e] - os[e]);"),
    "bwd_dv_without_alpha": ("dvu[e] += lw[nu] * a * g[e];", "dvu[e] += lw[nu] * g[e];"),
    "numerator_transposed_H": ("num += pq[c] * Hi[(size_t)c * d + e];", "num += pq[c] * Hi[(size_t)e * d + c];"),
}

# pins to run against a mutant (function, args after the oracle module)
PINS = [
    (pins.test_e4m3_encode_vs_torch_rne, ()),
    (pins.test_topk_count_table, ()),
    (pins.test_router_planted_scores, (True,)),
    (pins.test_router_projection_orientation, ("q",)),
    (pins.test_router_ties_go_to_lower_index, ()),
    (pins.test_all_blocks_alpha1_is_dense_attention, ("f32", 700, 64, 128)),
    (pins.test_row_mass_identity, ()),
    (pins.test_no_blocks_alpha0_is_linear_attention, ("f32", 700, 64)),
    (pins.test_linear_branch_over_unselected_blocks, ()),
    (pins.test_combine_is_alpha_mix_of_the_two_branches, ()),
    (pins.test_combine_alpha_per_query_block, ()),
    (pins.test_lowbit_identity_quantiser_equals_exact, ("bf16",)),
    (pins.test_lowbit_quantised_inputs, ()),
    (pins.test_lowbit_error_is_small, ()),
    (pins.test_lowbit_single_tile_closed_form, ()),
    (pins.test_lowbit_branch_and_flip_bound_brute_force, ()),
    (pins.test_lowbit_v_codes_and_scales_vs_torch, ()),
    (pins.test_lowbit_v_identity_quantiser_equals_exact, ()),
    (pins.test_lowbit_v_single_tile_closed_form, ()),
    (pins.test_lowbit_v_constant_v, ()),
    (pins.test_i8_encode_vs_torch_round, ()),
    (pins.test_lowbit_i8_quantised_inputs, ()),
    (pins.test_lowbit_i8_identity_quantiser_equals_exact, ()),
    (pins.test_lowbit_i8_single_tile_closed_form, (0,)),
    (pins.test_phi_softmax_linear_attention, ("f32",)),
    (pins.test_v1_negligible_count_table, ()),
    (pins.test_v1_router_brute_force, ()),
    (pins.test_v1_is_sparse_plus_projected_linear, (1,)),
    (pins.test_v1_all_marginal_or_none, ()),
    (pins.test_soft_topk_keeps_the_budget, (5,)),
    (pins.test_soft_topk_gradient_vs_finite_differences, ()),
    (pins.test_route_grad_vs_finite_differences, ()),
    (pins.test_backward_vs_torch_autograd, (0, 0, 0.4)),
    (pins.test_backward_vs_finite_differences, ()),
]


def _load_mutant(tmp_path, name, find, repl):
    src = open(SRC).read()
    assert src.count(find) == 1, f"mutation anchor for {name} not unique"
    mdir = tmp_path / name
    mdir.mkdir()
    c = mdir / "sla2_oracle.c"
    c.write_text(src.replace(find, repl))
    so = mdir / "libsla2_oracle.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-w",
                           "-o", str(so), str(c), "-lm"])
    spec = importlib.util.spec_from_file_location(f"oracle_mut_{name}",
                                                  os.path.join(ROOT, "oracle", "oracle.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod._LIB = str(so)
    mod._lib = None
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(tmp_path, name):
    find, repl = MUTANTS[name]
    mod = _load_mutant(tmp_path, name, find, repl)
    caught = []
    for fn, args in PINS:
        try:
            fn(mod, *args)
        except AssertionError:
            caught.append(fn.__name__)
    assert caught, f"no pin caught the planted mistake {name!r}"


def test_unmutated_copy_passes(tmp_path):
    mod = _load_mutant(tmp_path, "none", "int orc_num_blocks(int n, int b)",
                       "int orc_num_blocks(int n, int b)")
    for fn, args in PINS:
        fn(mod, *args)
