"""Plant one plausible mistake at a time into a copy of oracle.c (on the CPU,
in a temporary directory) and check that the pin suite fails on it.  This
shows the pins are sharp enough to catch a dropped term, a wrong sign, a
wrong index or a wrong rounding."""
import os
import subprocess
import sys

import pytest

from oracle import build as obuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "eps_dropped": ("ss / (double)H + eps", "ss / (double)H"),
    "mean_over_H_minus_1": ("sqrt(ss / (double)H + eps)", "sqrt(ss / (double)(H - 1) + eps)"),
    "rsqrt_missing": ("1.0 / sqrt(ss / (double)H + eps)", "1.0 / (ss / (double)H + eps)"),
    "dx_sign": ("w[j] * dy[j] - xhat * c", "w[j] * dy[j] + xhat * c"),
    "dx_c_term_dropped": ("w[j] * dy[j] - xhat * c", "w[j] * dy[j]"),
    "dx_outer_rho_dropped": ("dx[j] = rho * (w[j] * dy[j] - xhat * c);", "dx[j] = (w[j] * dy[j] - xhat * c);"),
    "row_dot_without_w": ("c += (u[j] * rho) * w[j] * dy[j];", "c += (u[j] * rho) * dy[j];"),
    "row_dot_not_averaged": ("c /= (double)H;", ""),
    "dres_dropped": ("if (dres) dx[j] += dres[j];", ""),
    "y_without_w_f64": ("y[r * H + j] = ur[j] * s * w[j];", "y[r * H + j] = ur[j] * s;"),
    "y_without_w_bf16": ("y[o + j] = oracle_bf16_round(u[j] * s * wd[j]);", "y[o + j] = oracle_bf16_round(u[j] * s);"),
    "dw_f64_index": ("acc += dy[r * H + j] * (u[r * H + j] * rho[r]);",
                     "acc += dy[r * H + j] * (u[r * H + (H - 1 - j)] * rho[r]);"),
    "dw_bf16_rho_dropped": ("(oracle_bf16_to_double(u16[row * H + j]) * rho);",
                            "(oracle_bf16_to_double(u16[row * H + j]));"),
    "dw_bf16_transposed_operand": ("acc[j - j0] += oracle_bf16_to_double(dy16[row * H + j])",
                                   "acc[j - j0] += oracle_bf16_to_double(u16[row * H + j])"),
    "round_ties_away": ("r = ldexp(rint(ldexp(m, 8)), e - 8);", "r = ldexp(floor(ldexp(m, 8) + 0.5), e - 8);"),
    "round_truncates": ("r = ldexp(rint(ldexp(m, 8)), e - 8);", "r = ldexp(trunc(ldexp(m, 8)), e - 8);"),
    "residual_sign": ("h[i] = oracle_bf16_round(oracle_bf16_to_double(x[i]) + oracle_bf16_to_double(r[i]));",
                      "h[i] = oracle_bf16_round(oracle_bf16_to_double(x[i]) - oracle_bf16_to_double(r[i]));"),
    "residual_not_normalised": ("u[j] = oracle_bf16_to_double(hb);", "u[j] = oracle_bf16_to_double(x[o + j]);"),
    # SiLU-gated variant
    "gate_dropped_f64_fwd": ("ur[j] * s * w[j] * silu(g[r * H + j])", "ur[j] * s * w[j]"),
    "gate_dropped_bf16_fwd": ("u[j] * s * wd[j] * silu(oracle_bf16_to_double(g[o + j]))", "u[j] * s * wd[j]"),
    "sigmoid_exponent_capped": ("static double sigmoid(double g) { return 1.0 / (1.0 + exp(-g)); }",
                                "static double sigmoid(double g) { return 1.0 / (1.0 + exp(fmin(-g, 87.0))); }"),
    "silu_is_identity": ("static double silu(double g) { return g * sigmoid(g); }",
                         "static double silu(double g) { return g; }"),
    "silu_grad_sign": ("return sg * (1.0 + g * (1.0 - sg));", "return sg * (1.0 - g * (1.0 - sg));"),
    "silu_grad_without_sigmoid": ("return sg * (1.0 + g * (1.0 - sg));", "return (1.0 + g * (1.0 - sg));"),
    "dg_without_w": ("dg[j] = dy[j] * ((u[j] * rho) * w[j]) * silu_grad(g[j]);",
                     "dg[j] = dy[j] * (u[j] * rho) * silu_grad(g[j]);"),
    "gated_dx_without_gate": ("e[j] = dy[j] * silu(g[j]);", "e[j] = dy[j];"),
    "gated_dw_f64_without_gate": ("acc += (dy[r * H + j] * silu(g[r * H + j])) * (u[r * H + j] * rho[r]);",
                                  "acc += dy[r * H + j] * (u[r * H + j] * rho[r]);"),
    "gated_dw_bf16_without_gate": ("silu(oracle_bf16_to_double(g16[row * H + j]));", "1.0;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(obuild.SRC).read()
    assert src.count(old) >= 1, f"anchor for {name} not found"
    path = tmp_path / "oracle_mutant.c"
    path.write_text(src.replace(old, new))
    lib = obuild.build(src=str(path), lib=str(tmp_path / "liboracle_mutant.so"))
    env = dict(os.environ, RMSNORM_ORACLE_LIB=lib)
    proc = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                           os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                           os.path.join(ROOT, "tests", "test_oracle_gated_pins.py")],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert proc.returncode != 0, f"mutant {name} passed every pin:\n{proc.stdout[-2000:]}"
