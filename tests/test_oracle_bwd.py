"""The fp64 MhcPre-backward oracle against its pins, and the pins against planted mistakes.

Every mutant is a textual change to oracle/mhc_oracle_bwd.c, compiled with gcc (beside
the unchanged forward source) into a temporary directory and run through every pin in
oracle_bwd_pins.py. A mutant that passes every pin would be a blind spot.
"""
import os
import subprocess

import pytest

import oracle
import oracle_bwd_pins

HERE = os.path.dirname(oracle.__file__)
SRC = os.path.join(HERE, "mhc_oracle_bwd.c")
FWD = os.path.join(HERE, "mhc_oracle.c")


@pytest.mark.parametrize("pin", oracle_bwd_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(None)


MUTANTS = {
    "pre_sigmoid_derivative_s": ("const double g2 = acc * s * (1.0 - s);", "const double g2 = acc * s;"),
    "pre_s_keeps_eps": ("const double s = (double)in->h_pre[t * n + i] - eps;",
                        "const double s = (double)in->h_pre[t * n + i];"),
    "post_derivative_without_half": ("hp * (1.0 - hp / 2.0)", "hp * (1.0 - hp)"),
    "alpha0_grad_unnormalised": ("ta[0] += g2 * ((double)in->h_mix[t * M + i] * inv);",
                                 "ta[0] += g2 * (double)in->h_mix[t * M + i];"),
    "alpha1_grad_uses_pre_rows": ("ta[1] += g2 * ((double)in->h_mix[t * M + n + i] * inv);",
                                  "ta[1] += g2 * ((double)in->h_mix[t * M + i] * inv);"),
    "res_grad_not_scaled": ("gw[2 * n + e] = g * a2;", "gw[2 * n + e] = g;"),
    "alpha2_grad_uses_hres_grad_squared": ("ta[2] += g * ((double)in->h_mix[t * M + 2 * n + e] * inv);",
                                           "ta[2] += g * g;"),
    "gmix_without_inv": ("gmix[m] = gw[m] * inv;", "gmix[m] = gw[m];"),
    "ginv_from_gmix": ("gi += gw[m] * (double)in->h_mix[t * M + m];",
                       "gi += gmix[m] * (double)in->h_mix[t * M + m];"),
    "rms_term_sign": ("const double vr = -c3 * xv;", "const double vr = c3 * xv;"),
    "rms_term_inv_squared": ("ginv[t] * inv * inv * inv / (double)K", "ginv[t] * inv * inv / (double)K"),
    "rms_term_over_D": ("ginv[t] * inv * inv * inv / (double)K", "ginv[t] * inv * inv * inv / (double)D"),
    "rms_term_on_x_rs": ("const double vr = -c3 * xv;", "const double vr = -c3 * xv * gk;"),
    "gamma_grad_without_x": ("sg += xv * xg;", "sg += xg;"),
    "phi_grad_without_gamma": ("const double xrs = xv * gk;", "const double xrs = xv;"),
    "mm_term_without_gamma": ("double g = v3 + mm * gk + vr;", "double g = v3 + mm + vr;"),
    "hin_branch_uses_hpost": ("const double hp = in->h_pre[t * n + i];", "const double hp = in->h_post[t * n + i];"),
    "x_post_dropped": ("g += gp;", "(void)gp;"),
    "phi_row_col_swapped": ("const double p = gmix[t * M + m] * (double)in->phi[(int64_t)m * K + k];",
                            "const double p = gmix[t * M + m] * (double)in->phi[(int64_t)(k % M) * K + (k / M) + m];"),
    "hpre_grad_reads_stream_0": ("x16_value(in, in->x[t * K + (int64_t)i * D + d]);",
                                 "x16_value(in, in->x[t * K + d]);"),
    "f16_inputs_read_as_bf16": ("return in->x_f16 ? oracle_f16_to_double(bits) : oracle_bf16_to_double(bits);",
                                "return oracle_bf16_to_double(bits);"),
    "f16_grad_x_rounded_to_bf16": ("return in->x_f16 ? oracle_f16_from_double(v) : oracle_bf16_from_double(v);",
                                   "return oracle_bf16_from_double(v);"),
    "sk_bwd_reads_previous_plane": ("const float* A = in->norm_out + ((int64_t)k * T + t) * n * n;",
                                    "const float* A = in->norm_out + ((int64_t)(k - 1) * T + t) * n * n;"),
    "sk_bwd_no_division": ("gl[e] = (gl[e] - u) / (double)sk[i];", "gl[e] = (gl[e] - u);"),
    "sk_bwd_rows_for_columns": ("const int e = (k % 2) ? j * n + i : i * n + j;\n                    u +=",
                                "const int e = (k % 2) ? i * n + j : j * n + i;\n                    u +="),
    "sk_bwd_softmax_keeps_eps": ("for (int c = 0; c < n; ++c) u += gl[r * n + c] * ((double)A0[r * n + c] - eps);",
                                 "for (int c = 0; c < n; ++c) u += gl[r * n + c] * (double)A0[r * n + c];"),
    "sk_bwd_skips_last_step": ("for (int k = 2 * in->num_iters - 1; k >= 1; --k) {",
                               "for (int k = 2 * in->num_iters - 2; k >= 1; --k) {"),
    "sk_bwd_no_softmax_step": ("            for (int c = 0; c < n; ++c) gl[r * n + c] = ((double)A0[r * n + c] - eps) * (gl[r * n + c] - u);",
                               "            (void)u;"),
    "fwd64_sinkhorn_sums_without_eps": ("double sum = eps;", "double sum = 0.0;"),
    "fwd64_res_unnormalised": ("alpha[2] * (hm[2 * n + e] * inv) + bias[2 * n + e]", "alpha[2] * hm[2 * n + e] + bias[2 * n + e]"),
    "fwd64_hin_uses_hpost_eps": ("hp[i] = sigm(alpha[0] * (hm[i] * inv) + bias[i]) + hc_eps;",
                                 "hp[i] = sigm(alpha[0] * (hm[i] * inv) + bias[i]);"),
}


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, source, tmp_path):
    old, new = MUTANTS[name]
    assert source.count(old) == 1, f"mutation site for {name} not unique / not found"
    c_path = tmp_path / "mutant_bwd.c"
    so_path = tmp_path / "libmutant.so"
    c_path.write_text(source.replace(old, new))
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-w",
                    "-o", str(so_path), FWD, str(c_path), "-lm"], check=True)
    lib = oracle.load_library(str(so_path))
    caught = []
    for pin in oracle_bwd_pins.ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutant {name}"
