"""Planted mistakes in the oracle must be caught by the pins.

Each mutant is a copy of oracle.c with one plausible mistake (a dropped term,
a wrong sign, index or divisor, a rounding mode), compiled on the CPU into a
temporary directory.  The pin battery of tests/pins.py must fail on every one
of them; the real oracle passes it (tests/test_oracle_pins.py).
"""
import os

import pytest

import oracle
import pins

LN_GAMMA = ("double g = gamma ? load_elem(gamma, i, dtype) : 1.0;\n"
            "                double b = beta")

# RMSNorm taken of the unrounded double sums instead of the stored h
UNROUNDED_NORM = """for (int64_t r = 0; r < M; ++r) {
        double q = 0.0;
        for (int64_t i = 0; i < N; ++i) {
            double v = load_elem(x, r * N + i, dtype) + load_elem(res, r * N + i, dtype);
            q += v * v;
        }
        double rs = 1.0 / sqrt(q / (double)N + eps);
        for (int64_t i = 0; i < N; ++i) {
            double g = gamma ? load_elem(gamma, i, dtype) : 1.0;
            double v = load_elem(x, r * N + i, dtype) + load_elem(res, r * N + i, dtype);
            if (y) y[r * N + i] = v * rs * g;
        }
        if (rstd) rstd[r] = rs;
    }
    return 0;"""

MUTANTS = {
    "unbiased_variance": ("double var = q / (double)N;", "double var = q / (double)(N - 1);"),
    "ln_eps_outside_root": ("double rs = 1.0 / sqrt(var + eps);", "double rs = 1.0 / sqrt(var) + eps;"),
    "ln_rstd_without_root": ("double rs = 1.0 / sqrt(var + eps);", "double rs = 1.0 / (var + eps);"),
    "ln_drop_beta": ("* rs * g + b;", "* rs * g;"),
    "ln_gamma_reversed": (LN_GAMMA, LN_GAMMA.replace("load_elem(gamma, i,", "load_elem(gamma, N - 1 - i,")),
    "ln_mean_sign": ("y[base + i] = (load_elem(x, base + i, dtype) - mu)",
                     "y[base + i] = (load_elem(x, base + i, dtype) + mu)"),
    "ln_naive_variance": ("double d = load_elem(x, base + i, dtype) - mu;\n            q += d * d;",
                          "double d = load_elem(x, base + i, dtype);\n            q += d * d - mu * mu;"),
    "ln_mean_divisor": ("double mu = s / (double)N;", "double mu = s / (double)(N + 1);"),
    "ln_row_stride": ("int64_t base = r * N;\n        double s = 0.0;",
                      "int64_t base = r * (N - 1);\n        double s = 0.0;"),
    "rms_drop_gamma": ("y[base + i] = load_elem(x, base + i, dtype) * rs * g;",
                       "y[base + i] = load_elem(x, base + i, dtype) * rs;"),
    "rms_eps_outside_root": ("double rs = 1.0 / sqrt(ms + eps);", "double rs = 1.0 / sqrt(ms) + eps;"),
    "rms_divisor": ("double ms = q / (double)N;", "double ms = q / (double)(N + 1);"),
    "round_truncates": ("double r = rint(k);", "double r = trunc(k);"),
    "f16_widen_bias": ("ex - 25", "ex - 24"),
    "bf16_widen_shift": ("(uint32_t)b << 16", "(uint32_t)b << 15"),
    "bf16_precision_off_by_one": ("rne_to_format(v, 8, -126)", "rne_to_format(v, 7, -126)"),
    "f16_min_normal_wrong": ("rne_to_format(a, 11, -14)", "rne_to_format(a, 11, -15)"),
    "add_residual_sign": ("double s = load_elem(x, i, dtype) + load_elem(res, i, dtype);",
                          "double s = load_elem(x, i, dtype) - load_elem(res, i, dtype);"),
    "add_residual_row0_broadcast": ("+ load_elem(res, i, dtype);", "+ load_elem(res, i % N, dtype);"),
    "add_residual_dropped": ("double s = load_elem(x, i, dtype) + load_elem(res, i, dtype);",
                             "double s = load_elem(x, i, dtype) + 0.0 * load_elem(res, i, dtype);"),
    "add_rms_norm_of_unrounded_sum": ("return oracle_rms_fwd(h, gamma, dtype, M, N, eps, y, rstd);",
                                      UNROUNDED_NORM),
    "fp8_scale_multiplies": ("double_to_e4m3_code(v[i] / scale)", "double_to_e4m3_code(v[i] * scale)"),
    "fp8_no_saturation": ("    if (a > 448.0)\n        a = 448.0;\n", ""),
    "fp8_exponent_bias_8": ("(e - 1 + 7) << 3", "(e - 1 + 8) << 3"),
    "fp8_subnormal_threshold": ("if (e - 1 < -6)", "if (e - 1 < -7)"),
    "fp8_precision_off_by_one": ("rne_to_format(a, 4, -6)", "rne_to_format(a, 3, -6)"),
    "bwd_gamma_outside_bracket": ("if (dx) dx[base + i] = rstd[r] * (g - gbar - xhat * gxbar);",
                                  "if (dx) dx[base + i] = (gamma ? load_elem(gamma, i, dtype) : 1.0) * rstd[r]"
                                  " * (d - gbar - xhat * gxbar);"),
    "bwd_missing_gbar": ("rstd[r] * (g - gbar - xhat * gxbar)", "rstd[r] * (g - xhat * gxbar)"),
    "bwd_xhat_term_sign": ("rstd[r] * (g - gbar - xhat * gxbar)", "rstd[r] * (g - gbar + xhat * gxbar)"),
    "bwd_dgamma_without_xhat": ("if (dgamma) dgamma[i] += d * xhat;", "if (dgamma) dgamma[i] += d;"),
    "bwd_dbeta_with_xhat": ("if (dbeta) dbeta[i] += d;", "if (dbeta) dbeta[i] += d * xhat;"),
    "bwd_gxbar_divisor": ("gxbar = sgx / (double)N;", "gxbar = sgx / (double)(N - 1);"),
    "rms_bwd_missing_x_term": ("if (dx) dx[base + i] = rs * g - xv * c;", "if (dx) dx[base + i] = rs * g;"),
    "rms_bwd_rstd_squared": ("double c = rs * rs * rs * sgx / (double)N;", "double c = rs * rs * sgx / (double)N;"),
    "rms_bwd_dgamma_without_rstd": ("if (dgamma) dgamma[i] += d * xv * rs;", "if (dgamma) dgamma[i] += d * xv;"),
    "add_rms_wrong_operand": ("double s = load_elem(x, i, dtype) + load_elem(res, i, dtype);",
                              "double s = load_elem(x, i, dtype) + load_elem(x, i, dtype);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle.SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    mpath = tmp_path / f"{name}.c"
    mpath.write_text(src.replace(old, new))
    lib = oracle.compile_c(str(mpath), str(tmp_path / f"lib{name}.so"))
    orc = oracle.Oracle(lib)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(orc)
        except Exception as e:          # AssertionError or a numeric failure
            caught.append(pin.__name__)
            break
    assert caught, f"no pin caught the planted mistake {name}"
