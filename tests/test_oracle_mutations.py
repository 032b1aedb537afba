"""The pins must catch plausible mistakes: each mutant below plants one
mistake in a copy of the oracle's C source (on the CPU, in a temp dir), and
the pin suite must fail against it."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "mhc_oracle.c")

MUTANTS = {
    "res_transposed": ("const float *r = res + (size_t)t * 16 + 4 * j;\n"
                       "                float a = r[0]",
                       "const float *r = res + (size_t)t * 16 + j;\n"
                       "                float a = r[0]"),
    "res_transposed_rest": ("a = fmaf(r[1], ", "a = fmaf(r[4], "),
    "post_term_dropped": ("a = fmaf(post[(size_t)t * 4 + j],\n"
                          "                         bf16_to_f32(y[(size_t)t * H + h]), a);",
                          "(void)0;"),
    "post_wrong_stream": ("post[(size_t)t * 4 + j]", "post[(size_t)t * 4 + (j ^ 1)]"),
    "collapse_wrong_stream": ("c = fmaf(p[2], xb[2 * (size_t)H + h], c);",
                              "c = fmaf(p[2], xb[1 * (size_t)H + h], c);"),
    "collapse_unrounded_residual": ("v = bf16_to_f32(b);", "v = a;"),
    "u_not_rounded": ("u[h] = bf16_to_f32(f32_to_bf16(c));", "u[h] = c;"),
    "eps_outside_root": ("float rstd_u = (float)(1.0 / sqrt(su / (double)H + (double)eps));",
                         "float rstd_u = (float)(1.0 / (sqrt(su / (double)H) + (double)eps));"),
    "sum_not_mean": ("sqrt(su / (double)H + ", "sqrt(su + "),
    "gate_mean_over_H": ("sqrt(ss / (double)K + ", "sqrt(ss / (double)H + "),
    "fn_transposed": ("(double)fn[r * 24 + k]", "(double)fn[(r % 24) * K / 24 + k * (K / 24) + 0 * r]"),
    "fn_interleaved_rows": ("d += (double)xb[r] * (double)fn[r * 24 + k];",
                            "d += (double)xb[(r % 4) * H + r / 4] * (double)fn[r * 24 + k];"),
    "sinkhorn_columns_first": ("for (int it = 0; it < iters; ++it) {\n        for (int j = 0; j < 4; ++j) {\n            double s = 0.0;\n            for (int i = 0; i < 4; ++i)\n                s += m[j][i];",
                               "for (int it = 0; it < iters; ++it) {\n        for (int j = 0; j < 4; ++j) {\n            double s = 0.0;\n            for (int i = 0; i < 4; ++i)\n                s += m[i][j];"),
    "sinkhorn_extra_iteration": ("for (int it = 0; it < iters; ++it) {\n        for (int j = 0; j < 4; ++j) {",
                                 "for (int it = 0; it <= iters; ++it) {\n        for (int j = 0; j < 4; ++j) {"),
    "sinkhorn_fixed_20_iterations": ("for (int it = 0; it < iters; ++it) {\n        for (int j = 0; j < 4; ++j) {",
                                     "for (int it = 0; it < 20; ++it) {\n        for (int j = 0; j < 4; ++j) {"),
    "sinkhorn_out_transposed": ("out16[4 * j + i] = m[j][i];", "out16[4 * j + i] = m[i][j];"),
    "post_gate_missing_2": ("(float)(2.0 * sigmoid(l[4 + j]))", "(float)(sigmoid(l[4 + j]))"),
    "pre_post_slices_swapped": ("(float)sigmoid(l[i]);", "(float)sigmoid(l[4 + i]);"),
    "bias_dropped": ("l[k] = rstd_g * d + (double)bias[k];", "l[k] = rstd_g * d;"),
    "e4m3_ties_away": ("if (hi < lo || (hi == lo && (c & 1)))", "if (hi <= lo)"),
    "scale_rule_floor": ("while (k < 127 && ldexp(448.0, k) < amax)", "while (k < 127 && ldexp(448.0, k + 1) < amax)"),
    "zero_group_scale": ("if (amax == 0.0)\n        return -127;", "if (amax == 0.0)\n        return 0;"),
    "bf16_truncates": ("return (uint16_t)((u + 0x7fffu + lsb) >> 16);", "return (uint16_t)(u >> 16);"),
    "grid_drops_scale": ("grid[idx] = f32_to_bf16((float)ldexp(q, k));", "grid[idx] = f32_to_bf16((float)q);"),
    "unshifted_uses_quarter_pre": ("collapse_norm(t, H, eps, pre_out + (size_t)t * 4, xb, gamma, norm, u);",
                                   "const float q4[4] = {0.25f, 0.25f, 0.25f, 0.25f};\n"
                                   "        collapse_norm(t, H, eps, q4, xb, gamma, norm, u);"),
    "unshifted_collapse_before_gates": ("        next_gates(t, H, eps, iters, xb, fn, bias, pre_out, post_out, res_out);\n"
                                        "        collapse_norm(t, H, eps, pre_out + (size_t)t * 4, xb, gamma, norm, u);",
                                        "        collapse_norm(t, H, eps, pre_out + (size_t)t * 4, xb, gamma, norm, u);\n"
                                        "        next_gates(t, H, eps, iters, xb, fn, bias, pre_out, post_out, res_out);"),
    "g128_scale_from_first_subgroup": ("for (int e = 0; e < G; ++e) {\n                double a = fabs(",
                                       "for (int e = 0; e < 32; ++e) {\n                double a = fabs("),
    "head_reduce_ignores_weights": ("collapse_row(H, w ? w + (size_t)t * 4 : quarter, xb, u);",
                                    "collapse_row(H, quarter, xb, u);"),
    "head_reduce_token_stride_H": ("xb[r] = bf16_to_f32(x[(size_t)t * 4 * H + r]);",
                                   "xb[r] = bf16_to_f32(x[(size_t)t * H + r]);"),
    "head_reduce_identity_sums": ("const float quarter[4] = {0.25f, 0.25f, 0.25f, 0.25f};\n#pragma omp parallel",
                                  "const float quarter[4] = {1.0f, 1.0f, 1.0f, 1.0f};\n#pragma omp parallel"),
    "gemm_unsigned_decode": ("e4m3_signed(a[(size_t)t * K + k]) * ea",
                             "e4m3_value(a[(size_t)t * K + k] & 0x7f) * ea"),
    "gemm_weights_as_k_by_n": ("(e4m3_signed(b[(size_t)n * K + k]) * eb)",
                               "(e4m3_signed(b[(size_t)k * N + n]) * eb)"),
    "gemm_scale_per_64": ("const double ea = e8m0_value(sa[(size_t)t * KB + kb]);",
                          "const double ea = e8m0_value(sa[(size_t)t * KB + kb / 2 * 2]);"),
    "gemm_scale_ff_as_power": ("return s == 0xff ? NAN : ldexp(1.0, s - 127);",
                               "return ldexp(1.0, s - 127);"),
    "fma_split": ("a = fmaf(r[3], bf16_to_f32(xt[3 * (size_t)H + h]), a);",
                  "a = r[3] * bf16_to_f32(xt[3 * (size_t)H + h]) + a;"),
}


@pytest.mark.slow
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mut = src.replace(old, new, 1)
    csrc = tmp_path / "mut.c"
    csrc.write_text(mut)
    lib = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp",
                    "-fPIC", "-shared", str(csrc), "-o", str(lib), "-lm"],
                   check=True)
    env = dict(os.environ, ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q",
                        "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode != 0, f"pins did not catch mutant {name}:\n{r.stdout[-2000:]}"
