"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that
the pins in test_oracle_pins.py catch every one of them.

Each mutant is a textual edit of h3oracle.c (the pattern must occur exactly
once), compiled with the same flags into a temporary library; the pin suite is
then run against it in a subprocess and must fail.
"""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "h3oracle.c")

MUTANTS = {
    "adaln_drop_one_plus_scale": ("xhat * (1.0 + sc) + sh", "xhat * sc + sh"),
    "adaln_swap_shift_scale": ("xhat * (1.0 + sc) + sh", "xhat * (1.0 + sh) + sc"),
    "adaln_unbiased_variance": ("const double var = ss / (double)D;",
                                "const double var = ss / (double)(D - 1);"),
    "adaln_eps_outside_sqrt": ("sqrt(var + eps)", "(sqrt(var) + eps)"),
    "gated_transposed": ("xv + gv * hv", "gv * xv + hv"),
    "swiglu_sign": ("a / (1.0 + exp(-a))", "a / (1.0 + exp(a))"),
    "swiglu_wrong_half": ("const double a = ld(gate_up, dtype, r * 2 * inner + j);",
                          "const double a = ld(gate_up, dtype, r * 2 * inner + inner + j);"),
    "rms_drop_eps": ("sqrt(ss / (double)Dh + eps)", "sqrt(ss / (double)Dh)"),
    "rms_wrong_weight": ("qk_head(k_out, k, k_weight,", "qk_head(k_out, k, q_weight,"),
    "rope_clockwise": ("u[e1] = a * sn + b * cs;", "u[e1] = -a * sn + b * cs;"),
    "rope_freq_exponent": ("pow(theta, -2.0 * (double)j / (double)dims[c])",
                           "pow(theta, -1.0 * (double)j / (double)dims[c])"),
    "rope_pairing": ("e0 = start + 2 * j;\n                e1 = start + 2 * j + 1;",
                     "e0 = start + j;\n                e1 = start + j + dc / 2;"),
    "rope_axis_order": ("const int32_t dims[3] = {d_t, d_h, d_w};\n    float inv_freq",
                        "const int32_t dims[3] = {d_w, d_h, d_t};\n    float inv_freq"),
    "positions_h_w_swapped": ("h = (int32_t)((p / W) % H);", "h = (int32_t)((p / H) % W);"),
    "audio_position_axis": ("t = (int32_t)(p - n_video);\n            h = 0;",
                            "t = 0;\n            h = (int32_t)(p - n_video);"),
    "bf16_round_half_up": ("u += 0x7fffu + lsb;", "u += 0x8000u + 0 * lsb;"),
    "affine_after_modulation": ("st(y, y_dtype, r * D + c, ln * (1.0 + sc) + sh);",
                                "st(y, y_dtype, r * D + c, (ln - ld(beta, mod_dtype, c)) * (1.0 + sc) + sh + ld(beta, mod_dtype, c));"),
    "affine_gamma_beta_swapped": ("const double ln = ld(gamma, mod_dtype, c) *", "const double ln = ld(beta, mod_dtype, c) *"),
    "subblock_sum_not_mean": ("= s / (double)(r1 - r0);", "= s;"),
    "subblock_full_block_divisor": ("= s / (double)(r1 - r0);", "= s / (double)block;"),
    "subblock_wrong_head": ("ld(x, dtype, (r * heads + h) * head_dim + d)",
                            "ld(x, dtype, (r * heads + 0) * head_dim + d)"),
    "subblock_scores_transposed": ("scores[((int64_t)h * nbq + i) * nbk + j] = s;",
                                   "scores[((int64_t)h * nbq + j) * nbk + i] = s;"),
    "subblock_keep_ceil": ("nb - (int64_t)floor(skipped)", "nb - (int64_t)ceil(skipped)"),
    "subblock_keep_step_off_by_one": ("if (step < first_step) return nb;",
                                      "if (step <= first_step) return nb;"),
    "subblock_select_smallest": ("if (a->score > b->score) return -1;\n    if (a->score < b->score) return 1;",
                                 "if (a->score > b->score) return 1;\n    if (a->score < b->score) return -1;"),
    "subblock_ties_higher_index": ("return (a->block > b->block) - (a->block < b->block);",
                                   "return (a->block < b->block) - (a->block > b->block);"),
    "group_by_modulo": ("return rows_per_group > 0 ? r / rows_per_group : 0;",
                        "return rows_per_group > 0 ? r % rows_per_group : 0;"),
    "residual_l1_den_of_cur": ("den += fabs(p);", "den += fabs(c);"),
    "residual_l1_squared": ("num += fabs(c - p);", "num += (c - p) * (c - p);"),
    "fused_ln_before_residual": (
        "gated_row(x, x_dtype, h, h_dtype, gate, r, g, hidden);\n"
        "        adaln_row(y, y_dtype, x, x_dtype, shift, scale, x_dtype, r, g, hidden,\n"
        "                  (double)eps);",
        "adaln_row(y, y_dtype, x, x_dtype, shift, scale, x_dtype, r, g, hidden,\n"
        "                  (double)eps);\n"
        "        gated_row(x, x_dtype, h, h_dtype, gate, r, g, hidden);"),
    "positions_offset_ignored": ("int64_t p = (token_offset + r) % L;", "int64_t p = r % L;"),
    "rope_chunk_start_fixed": ("start += dc;", "start += 0;"),
    "subblock_kept_unsorted": ("qsort(out, (size_t)keep, sizeof *out, by_index_asc);",
                               "(void)by_index_asc;"),
    "gated_gate_in_h_dtype": ("const double gv = ld(gate, x_dtype, g * D + c);",
                              "const double gv = ld(gate, h_dtype, g * D + c);"),
    "affine_drop_eps": ("const double sigma = sqrt(ss / (double)D + eps);",
                        "const double sigma = sqrt(ss / (double)D);"),
    "subblock_scores_half_dot": ("for (int32_t d = 0; d < head_dim; ++d) s += a[d] * c[d];",
                                 "for (int32_t d = 0; d < head_dim / 2; ++d) s += a[d] * c[d];"),
    "rope_exact_angle_exponent": ("phi = (double)p3[c] * pow(theta, -2.0 * (double)j / (double)dc);",
                                  "phi = (double)p3[c] * pow(theta, -1.0 * (double)j / (double)dc);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation pattern for {name} must occur exactly once"
    mutated = src.replace(old, new)
    csrc = tmp_path / "h3oracle.c"
    csrc.write_text(mutated)
    hdr = os.path.join(ROOT, "oracle")
    lib = tmp_path / "liboracle_mutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    "-I", hdr, "-o", str(lib), str(csrc), "-lm"], check=True)
    env = dict(os.environ, H3_ORACLE_LIB_OVERRIDE=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
