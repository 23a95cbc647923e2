"""Plant plausible mistakes in copies of the oracle and check the pins catch each one.

Every mutant is a textual change to oracle/mhc_oracle.c, compiled with gcc into a
temporary directory (CPU only) and run through all pins in oracle_pins.py. A
mutant that passes every pin would be a blind spot of the pins, and fails this test.
"""
import os
import subprocess

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "mhc_oracle.c")
BWD = os.path.join(os.path.dirname(oracle.__file__), "mhc_oracle_bwd.c")   # built beside it, unchanged

MUTANTS = {
    "rms_mean_over_D": ("ss / (double)K + norm_eps", "ss / (double)D + norm_eps"),
    "rms_without_norm_eps": ("sqrt(ss / (double)K + norm_eps)", "sqrt(ss / (double)K)"),
    "rms_on_x_squared_twice": ("ss += v * v;", "ss += v * v * v * v;"),
    # reading R2: invRms of raw x, not of the gamma-scaled x the projection uses
    "rms_on_gamma_scaled_x": ("    const double inv_rms = token_inv_rms(c, xt, c->n, c->D, c->norm_eps);",
                              "    double inv_rms; { double ss = 0.0; for (int64_t k = 0; k < K; ++k) {"
                              " double v = x_val(c, xt[k]) * (gamma ? (double)gamma[k] : 1.0); ss += v * v; }"
                              " inv_rms = 1.0 / sqrt(ss / (double)K + c->norm_eps); }"),
    "gamma_indexed_by_d_only": ("if (gamma) xg *= (double)gamma[k];", "if (gamma) xg *= (double)gamma[k % c->D];"),
    "phi_transposed": ("acc += xg * (double)row[k];", "acc += xg * (double)phi[k * M + m]; (void)row;"),
    "w_not_normalised": ("double p_pre = hmix[i] * inv_rms;", "double p_pre = hmix[i];"),
    "hpre_without_eps": ("hpre[i] = sigmoid((double)alpha[0] * p_pre + (double)bias[i]) + eps;",
                         "hpre[i] = sigmoid((double)alpha[0] * p_pre + (double)bias[i]);"),
    "hpost_uses_alpha0": ("2.0 * sigmoid((double)alpha[1] * p_post", "2.0 * sigmoid((double)alpha[0] * p_post"),
    "hpost_uses_pre_bias": ("+ (double)bias[n + i]);", "+ (double)bias[i]);"),
    "hpost_eps_always": ("if (c->n_alpha == 2) hpost[i] += eps;", "hpost[i] += eps;"),
    "hpost_missing_factor_2": ("hpost[i] = 2.0 * sigmoid(", "hpost[i] = 1.0 * sigmoid("),
    "sigmoid_sign": ("if (z >= 0.0) return 1.0 / (1.0 + exp(-z));", "if (z >= 0.0) return 1.0 / (1.0 + exp(z));"),
    "res_bias_transposed": ("+ (double)bias[2 * n + m];", "+ (double)bias[2 * n + cc * n + r];"),
    "res_uses_alpha1": ("A[m] = (double)alpha[2] *", "A[m] = (double)alpha[1] *"),
    "softmax_without_eps": ("A[r * n + cc] = A[r * n + cc] / sum + eps;", "A[r * n + cc] = A[r * n + cc] / sum;"),
    "softmax_not_stabilised": ("A[r * n + cc] = exp(A[r * n + cc] - mx);", "A[r * n + cc] = exp(A[r * n + cc]); (void)mx;"),
    "row_col_order_swapped": ("} else if (k % 2 == 1) {", "} else if (k % 2 == 0) {"),
    "column_sum_without_eps": ("for (int r = 0; r < n; ++r) sum += A[r * n + cc];\n                    sum += eps;",
                               "for (int r = 0; r < n; ++r) sum += A[r * n + cc];"),
    "one_step_short": ("for (int k = 0; k < steps; ++k) {", "for (int k = 0; k < steps - 1; ++k) {"),
    "hin_weights_hpost": ("wgt[i] = pre_mix ? (double)pre_mix[t * n + i] : hpre[i];",
                          "wgt[i] = pre_mix ? (double)pre_mix[t * n + i] : hpost[i];"),
    "hin_reads_interleaved_x": ("x_val(c, xt[(int64_t)i * D + d]);",
                                "x_val(c, xt[(int64_t)d * n + i]);"),
    "hin_on_normalised_x": ("acc += wgt[i] * x_val(c, xt[(int64_t)i * D + d]);",
                            "acc += wgt[i] * inv_rms * x_val(c, xt[(int64_t)i * D + d]);"),
    "bf16_ties_away": ("else qr = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;", "else qr = fl + 1.0;"),
    "bf16_truncates": ("if (diff > 0.5) qr = fl + 1.0;", "if (diff > 2.0) qr = fl + 1.0;"),
}


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, source, tmp_path):
    old, new = MUTANTS[name]
    assert source.count(old) == 1, f"mutation site for {name} not unique / not found"
    mutated = source.replace(old, new)
    c_path = tmp_path / "mutant.c"
    so_path = tmp_path / "libmutant.so"
    c_path.write_text(mutated)
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-w",
                    "-o", str(so_path), str(c_path), BWD, "-lm"], check=True)
    lib = oracle.load_library(str(so_path))
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutant {name}"
