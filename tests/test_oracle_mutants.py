"""The oracle's pins catch plausible mistakes.

Each case plants one mistake (a flipped sign, a wrong index or frequency, a dropped
term, a transposed operand, the diagonal left out of the causal mask, a gradient
formula gone wrong) in a copy of
the oracle's C source, builds it in a temporary directory, routes the oracle module
to it and checks that at least one pin of ``test_oracle_pins`` fails.  CPU only.
"""
import os
import shutil
import subprocess

import pytest

import oracle
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "la_oracle.c")

MUTANTS = {
    "rope_sign": ("out[i] = x0 * c - x1 * s;", "out[i] = x0 * c + x1 * s;"),
    "rope_frequency": ("pow(base, -2.0 * (double)i / (double)D)", "pow(base, -1.0 * (double)i / (double)D)"),
    "rope_interleaved_pairs": ("double x0 = x[i], x1 = x[i + half];",
                               "double x0 = x[2 * i], x1 = x[2 * i + 1];"),
    "rmsnorm_sum_not_mean": ("double r = sqrt(ss / (double)D + eps);", "double r = sqrt(ss + eps);"),
    "rmsnorm_eps_dropped": ("double r = sqrt(ss / (double)D + eps);", "double r = sqrt(ss / (double)D);"),
    "sigmoid_sign": ("return 1.0 / (1.0 + exp(-x));", "return 1.0 / (1.0 + exp(x));"),
    "k_position_off_by_one": ("prologue_row(k + row, D, pos0 + t, base, eps, k_w, tmp, kh);",
                              "prologue_row(k + row, D, pos0 + t + 1, base, eps, k_w, tmp, kh);"),
    "state_transposed_in_readout": ("for (int i = 0; i < D; ++i) u += qh[i] * Sbh[i * D + j];",
                                    "for (int i = 0; i < D; ++i) u += qh[i] * Sbh[j * D + i];"),
    "diagonal_excluded": (
        "      /* S_t = S_{t-1} + k_t v_t^T  (columns j0..j1 of this task) */\n"
        "      for (int i = 0; i < D; ++i)\n"
        "        for (int j = j0; j < j1; ++j) Sbh[i * D + j] += kh[i] * (double)v[row + j];\n",
        "      for (int j = j0; j < j1; ++j) {\n"
        "        double u = 0.0;\n"
        "        for (int i = 0; i < D; ++i) u += qh[i] * Sbh[i * D + j];\n"
        "        o[row + j] = sigmoid((double)g[row + j]) * u;\n"
        "      }\n"
        "      for (int i = 0; i < D; ++i)\n"
        "        for (int j = j0; j < j1; ++j) Sbh[i * D + j] += kh[i] * (double)v[row + j];\n"
        "      continue;\n"),
    "update_uses_q_not_k": ("Sbh[i * D + j] += kh[i] * (double)v[row + j];",
                            "Sbh[i * D + j] += qh[i] * (double)v[row + j];"),
    "chunk_mask_strict": ("for (int s = 0; s <= r; ++s) {", "for (int s = 0; s < r; ++s) {"),
    "chunk_prefix_term_dropped": (
        "          for (int i = 0; i < D; ++i) u += qh[(int64_t)r * D + i] * Sbh[i * D + j];\n", "\n"),
    # gradients
    "back_rope_not_inverted": ("dn[i] = dy[i] * c + dy[i + half] * s;", "dn[i] = dy[i] * c - dy[i + half] * s;"),
    "back_rmsnorm_jacobian_term_dropped": (
        "dx[i] = wi * dn[i] / r - (double)x[i] * dot / ((double)D * r * r * r);", "dx[i] = wi * dn[i] / r;"),
    "back_sigmoid_derivative": ("dg[row + j] = (double)dout[row + j] * u * sg * (1.0 - sg);",
                                "dg[row + j] = (double)dout[row + j] * u * sg;"),
    "back_state_gradient_after_use": (
        "      for (int i = 0; i < D; ++i)\n"
        "        for (int j = 0; j < D; ++j) G[(size_t)i * D + j] += qh[(int64_t)t * D + i] * du[(int64_t)t * D + j];\n"
        "      for (int i = 0; i < D; ++i) {\n"
        "        double a = 0.0;\n"
        "        for (int j = 0; j < D; ++j) a += G[(size_t)i * D + j] * (double)v[row + j];\n"
        "        dkh[(int64_t)t * D + i] = a;\n"
        "      }\n",
        "      for (int i = 0; i < D; ++i) {\n"
        "        double a = 0.0;\n"
        "        for (int j = 0; j < D; ++j) a += G[(size_t)i * D + j] * (double)v[row + j];\n"
        "        dkh[(int64_t)t * D + i] = a;\n"
        "      }\n"
        "      for (int i = 0; i < D; ++i)\n"
        "        for (int j = 0; j < D; ++j) G[(size_t)i * D + j] += qh[(int64_t)t * D + i] * du[(int64_t)t * D + j];\n"),
    "back_dv_uses_q": ("for (int i = 0; i < D; ++i) a += kh[(int64_t)t * D + i] * G[(size_t)i * D + j];",
                       "for (int i = 0; i < D; ++i) a += qh[(int64_t)t * D + i] * G[(size_t)i * D + j];"),
    "back_weight_gradient_missing_norm": ("if (dw) dw[i] += dn[i] * (double)x[i] / r;",
                                          "if (dw) dw[i] += dn[i] * (double)x[i];"),
}

PIN_CALLS = [
    (pins.test_rmsnorm_closed_forms, ()),
    (pins.test_rmsnorm_invariants, ()),
    (pins.test_rope_d2_is_complex_rotation, ()),
    (pins.test_rope_d4_basis_vectors_fix_frequencies_and_pairing, ()),
    (pins.test_rope_identity_norm_and_relative_property, ()),
    (pins.test_recurrence_equals_bruteforce_quadratic, (2, 37, 3, 8, 1000, True)),
    (pins.test_recurrence_equals_bruteforce_quadratic, (1, 64, 1, 128, 262144, True)),
    (pins.test_hand_worked_example, ()),
    (pins.test_state_closed_form_and_independence_from_q_and_gate, ()),
    (pins.test_gate_special_cases, ()),
    (pins.test_chunked_equals_recurrence_for_every_chunk_size, ()),
    (pins.test_backward_matches_finite_differences, (True,)),
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    mutant = tmp_path / "la_oracle_mutant.c"
    mutant.write_text(src.replace(old, new, 1))
    lib = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", str(mutant),
                           "-o", str(lib), "-lm"])
    caught = None
    with oracle.use_library(str(lib)):
        for fn, args in PIN_CALLS:
            try:
                fn(*args)
            except AssertionError:
                caught = fn.__name__
                break
    assert caught is not None, f"no pin caught the planted mistake {name}"
