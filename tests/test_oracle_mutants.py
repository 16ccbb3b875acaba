"""Plant plausible mistakes in a copy of the oracle's C source (on the CPU) and check
that the pins in test_oracle_pins.py, test_oracle_bwd_pins.py, test_oracle_conv_pins.py and
test_oracle_proj_pins.py catch every one."""
import os
import shutil

import numpy as np
import pytest

import oracle
from tests import test_oracle_bwd_pins as bpins
from tests import test_oracle_conv_pins as cpins
from tests import test_oracle_pins as pins
from tests import test_oracle_proj_pins as ppins

SRC = os.path.join(os.path.dirname(oracle.__file__), "ss_oracle.c")

# (name, [(original text, planted text), ...]) -- each original must occur in the source;
# its first occurrence is replaced
MUTANTS = [
    ("drop_D_term", [("double yv = acc + D_d * uv;", "double yv = acc;")]),
    ("bias_after_softplus", [("const double x = in_at(delta, dtype, e) + bias_d;",
                              "const double x = in_at(delta, dtype, e);"),
                             ("const double dt = softplus_flag ? softplus(x) : x;",
                              "const double dt = (softplus_flag ? softplus(x) : x) + bias_d;")]),
    ("no_softplus", [("const double dt = softplus_flag ? softplus(x) : x;", "const double dt = x;")]),
    ("y_reads_old_state", [("      h[n] = abar * h[n] + (bbar * in_at(B, dtype, bc + n)) * uv;\n"
                            "      acc += in_at(C, dtype, bc + n) * h[n];",
                            "      acc += in_at(C, dtype, bc + n) * h[n];\n"
                            "      h[n] = abar * h[n] + (bbar * in_at(B, dtype, bc + n)) * uv;")]),
    ("A_transposed", [("(double)A[d * dstate + n]", "(double)A[n * dim + d]")]),
    ("B_C_swapped", [("(bbar * in_at(B, dtype, bc + n))", "(bbar * in_at(C, dtype, bc + n))"),
                     ("acc += in_at(C, dtype, bc + n) * h[n];", "acc += in_at(B, dtype, bc + n) * h[n];")]),
    ("decay_sign", [("const double abar = exp(dt * a_dn);", "const double abar = exp(-dt * a_dn);")]),
    ("input_term_without_dt", [("const double bbar = !zoh ? dt :", "const double bbar = !zoh ? 1.0 :")]),
    ("zoh_not_divided_by_A", [("expm1(dt * a_dn) / a_dn : dt", "expm1(dt * a_dn) : dt")]),
    ("zoh_zero_A_limit", [("expm1(dt * a_dn) / a_dn : dt", "expm1(dt * a_dn) / a_dn : 0.0")]),
    ("zoh_ignored", [("const double bbar = !zoh ? dt :", "const double bbar = 1 ? dt :")]),
    ("zoh_sign", [("expm1(dt * a_dn) / a_dn : dt", "-expm1(dt * a_dn) / a_dn : dt")]),
    ("zoh_divides_by_dt_A", [("expm1(dt * a_dn) / a_dn : dt", "expm1(dt * a_dn) / (dt * a_dn) : dt")]),
    ("gate_skips_D_term", [("    double yv = acc + D_d * uv;\n    if (z) yv *= silu(in_at(z, dtype, e));",
                            "    double yv = acc;\n    if (z) yv *= silu(in_at(z, dtype, e));\n    yv += D_d * uv;")]),
    ("gate_is_sigmoid", [("if (z >= 0.0) return z / (1.0 + exp(-z));", "if (z >= 0.0) return 1.0 / (1.0 + exp(-z));"),
                         ("return z * e / (1.0 + e);", "return e / (1.0 + e);")]),
    ("B_one_token_late", [("      h[n] = abar * h[n] + (bbar * in_at(B, dtype, bc + n)) * uv;\n",
                           "      h[n] = abar * h[n] + (bbar * in_at(B, dtype, (t > 0 ? bc - dstate : bc) + n)) * uv;\n")]),
    ("B_ignores_batch", [("const int64_t bc = (b * seqlen + t) * dstate;", "const int64_t bc = t * dstate;")]),
    ("bf16_decode_shift", [("<< 16;", "<< 15;")]),
    ("state_not_carried_in_step", [("state + j * dstate, y ? y + j : NULL, 1);",
                                    "state + 0 * dstate, y ? y + j : NULL, 1);")]),
    # backward
    ("bwd_carry_without_decay", [("mu[n] = abar * lam;", "mu[n] = lam;")]),
    ("bwd_ddt_drops_decay_term", [("ddt += lam * Bv * uv + g_abar * abar * a_dn;", "ddt += lam * Bv * uv;")]),
    ("bwd_no_softplus_derivative", [("const double dx = softplus_flag ? ddt * sigmoid(x) : ddt;",
                                     "const double dx = ddt;")]),
    ("bwd_dB_without_dt", [("dB[bc + n] += lam * dt * uv;", "dB[bc + n] += lam * uv;")]),
    ("bwd_dC_from_previous_state", [("dC[bc + n] += ds * ht[n];", "dC[bc + n] += ds * hp[n];")]),
    ("bwd_dsilu_is_sigmoid", [("return s * (1.0 + z * (1.0 - s));", "return s;")]),
    ("bwd_dA_without_dt", [("dA_ch[n] += g_abar * abar * dt;", "dA_ch[n] += g_abar * abar;")]),
    ("bwd_dlast_ignored", [("mu[n] = dlast_ch ? (double)dlast_ch[n] : 0.0;", "mu[n] = 0.0;")]),
    ("bwd_du_without_D", [("double du_t = ds * D_d;", "double du_t = 0.0;")]),
    ("bwd_decay_grad_uses_current_state", [("const double g_abar = lam * hp[n];", "const double g_abar = lam * ht[n];")]),
    ("bwd_gate_not_applied", [("      ds = dyv * silu(zv);\n", "      ds = dyv;\n")]),
    # conv prologue
    ("conv_filter_not_flipped", [("pre += (double)conv_w[d * kconv + m] * xv;",
                                  "pre += (double)conv_w[d * kconv + (kconv - 1 - m)] * xv;")]),
    ("conv_no_bias", [("double pre = conv_b ? (double)conv_b[d] : 0.0;", "double pre = 0.0;")]),
    ("conv_no_silu", [("u[(b * seqlen + t) * dim + d] = silu(pre);", "u[(b * seqlen + t) * dim + d] = pre;")]),
    ("conv_state_ignored", [("else xv = conv_state ? (double)conv_state[(b * dim + d) * (kconv - 1) + (kconv - 1) + tau] : 0.0;",
                             "else xv = 0.0;")]),
    ("conv_state_reversed", [("(double)conv_state[(b * dim + d) * (kconv - 1) + (kconv - 1) + tau]",
                              "(double)conv_state[(b * dim + d) * (kconv - 1) - 1 - tau]")]),
    ("conv_acausal", [("const int64_t tau = t - (kconv - 1) + m;", "const int64_t tau = t + m;")]),
    # input projections
    ("proj_B_C_swapped", [("B[bt * dstate + n] = xp[rank + n];", "B[bt * dstate + n] = xp[rank + dstate + n];"),
                          ("C[bt * dstate + n] = xp[rank + dstate + n];", "C[bt * dstate + n] = xp[rank + n];")]),
    ("proj_Wx_transposed", [("in_at(W_x, w_dtype, o * dim + d)", "in_at(W_x, w_dtype, d * nx + o)")]),
    ("proj_Wdt_transposed", [("in_at(W_dt, w_dtype, d * rank + r)", "in_at(W_dt, w_dtype, r * dim + d)")]),
    ("proj_B_off_by_one", [("B[bt * dstate + n] = xp[rank + n];", "B[bt * dstate + n] = xp[rank - 1 + n];")]),
    ("proj_step_from_inputs", [("acc += in_at(W_dt, w_dtype, d * rank + r) * xp[r];",
                                "acc += in_at(W_dt, w_dtype, d * rank + r) * in_at(u, u_dtype, ub + r);")]),
]


def pin_suite(lib):
    """Run the pins against ``lib``; return the names of the pins that fail."""
    failed = []
    checks = [
        ("brute", lambda: pins.test_brute_force_unrolled_sum(lib, True, True)),
        ("brute_ungated", lambda: pins.test_brute_force_unrolled_sum(lib, False, True)),
        ("brute_no_softplus", lambda: pins.test_brute_force_no_softplus_no_bias(lib)),
        ("brute_bf16", lambda: pins.test_brute_force_bf16_inputs(lib)),
        ("conv", lambda: pins.test_lti_equals_convolution(lib, True)),
        ("geometric", lambda: pins.test_geometric_series_constant_inputs(lib)),
        ("zero_step", lambda: pins.test_zero_step_keeps_state_exactly(lib)),
        ("huge_step", lambda: pins.test_huge_step_resets_state(lib)),
        ("page5", lambda: pins.test_page5_worked_example(lib)),
        ("page5_selective", lambda: pins.test_page5_selective_example(lib)),
        ("step", lambda: pins.test_step_by_step_matches_forward(lib)),
        ("zoh_continuous", lambda: pins.test_zoh_matches_continuous_solution(lib)),
        ("zoh_half_steps", lambda: pins.test_zoh_half_steps_compose(lib)),
        ("zoh_brute", lambda: pins.test_zoh_brute_force_unrolled_sum(lib, True)),
        ("zoh_step", lambda: pins.test_zoh_step_by_step_matches_forward(lib)),
        ("bwd_fd", lambda: bpins.test_backward_matches_finite_differences(lib, True)),
        ("bwd_fd_no_softplus", lambda: bpins.test_backward_matches_finite_differences(lib, False)),
        ("bwd_adjoint_u", lambda: bpins.test_adjoint_identity_for_linear_arguments(lib, "u")),
        ("bwd_adjoint_h0", lambda: bpins.test_adjoint_identity_for_linear_arguments(lib, "h0")),
        ("bwd_lti", lambda: bpins.test_lti_du_is_correlation_with_kernel(lib)),
        ("bwd_zero_step", lambda: bpins.test_zero_step_closed_forms(lib)),
        ("conv_numpy", lambda: cpins.test_conv_matches_numpy_convolve(lib, 4, True, True)),
        ("conv_impulse", lambda: cpins.test_impulse_response(lib)),
        ("conv_split", lambda: cpins.test_split_continues_with_conv_state(lib)),
        ("proj_numpy", lambda: ppins.test_matches_numpy_product_other_association(lib)),
        ("proj_selection", lambda: ppins.test_selection_matrices_are_exact(lib)),
        ("proj_rank1", lambda: ppins.test_rank_one_closed_form(lib)),
    ]
    for name, fn in checks:
        try:
            fn()
        except AssertionError:
            failed.append(name)
    return failed


def test_unmodified_copy_passes(tmp_path):
    src = tmp_path / "ss_oracle.c"
    shutil.copy(SRC, src)
    lib = oracle.Library(oracle.compile_source(str(src), str(tmp_path / "lib.so")))
    assert pin_suite(lib) == []


@pytest.mark.parametrize("name,edits", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, edits):
    text = open(SRC).read()
    for old, new in edits:
        # the forward loop comes first in the file; the backward repeats a few of its lines
        # for its own recomputation, and a forward mistake is planted in the forward only
        assert text.count(old) >= 1, f"mutation anchor not found: {old!r}"
        text = text.replace(old, new, 1)
    src = tmp_path / "ss_oracle_mutant.c"
    src.write_text(text)
    lib = oracle.Library(oracle.compile_source(str(src), str(tmp_path / "mutant.so")))
    failed = pin_suite(lib)
    assert failed, f"planted mistake {name} passed every pin"
