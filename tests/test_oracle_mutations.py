"""The pins must catch plausible mistakes in the oracle.

Each case plants one mistake in a copy of ``oracle/ss_oracle.c`` (on the
CPU, in a temporary directory), builds it, and runs the pin suites against
that copy in a subprocess; the suites must fail.  The real oracle is never
modified.
"""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "ss_oracle.c")

MUTATIONS = {
    "decay_sign_flipped": ("double abar = exp(dt * A[d * ns + n]);\n                double bt",
                           "double abar = exp(-dt * A[d * ns + n]);\n                double bt"),
    "B_index_transposed": ("double bt = B[(b * ns + n) * nl + t];\n                h[n]",
                           "double bt = B[(b * nl + t) * ns + n];\n                h[n]"),
    "C_index_transposed": ("acc += C[(b * ns + n) * nl + t] * h[n];",
                           "acc += C[(b * nl + t) * ns + n] * h[n];"),
    "skip_term_dropped": ("double ypre = acc + (D ? D[d] * ut : 0.0);\n            if (z) {\n                double zt",
                          "double ypre = acc;\n            if (z) {\n                double zt"),
    "bias_ignored": ("double x = raw + (bias ? bias[d] : 0.0);", "double x = raw;"),
    "softplus_unstable_branch": ("return (x > 0 ? x : 0.0) + log1p(exp(-ax));",
                                 "return (x > 0 ? x : 0.0) + log1p(exp(-x));"),
    "input_term_missing_delta": ("h[n] = abar * h[n] + dt * bt * ut;", "h[n] = abar * h[n] + bt * ut;"),
    "ddelta_drops_Bu": ("d_dt += g[n] * (a * abar * h_prev[n] + bt * ut);",
                        "d_dt += g[n] * (a * abar * h_prev[n]);"),
    "dA_drops_decay": ("dA[d * ns + n] += g[n] * dl[t] * abar * h_prev[n];",
                       "dA[d * ns + n] += g[n] * dl[t] * h_prev[n];"),
    "dC_uses_previous_state": ("dC[(b * ns + n) * nl + t] += dy * h_t[n];",
                               "dC[(b * ns + n) * nl + t] += dy * h_prev[n];"),
    "adjoint_carry_missing": ("g[n] *= abar;                             /* carried to t-1 */",
                              "g[n] *= 1.0;"),
    "gate_derivative_wrong": ("dz[r * nl + t] = dout_t * ypre * s * (1.0 + zt * (1.0 - s));",
                              "dz[r * nl + t] = dout_t * ypre * s * (1.0 + zt * s);"),
    "softplus_grad_missing": ("raw_grad *= sso_sigmoid(delta[r * nl + t] + (bias ? bias[d] : 0.0));",
                              "raw_grad *= 1.0;"),
    "state_update_B_batch_ignored": ("*h = abar * *h + dt * B[b * ns + n] * ut;",
                                     "*h = abar * *h + dt * B[n] * ut;"),
    "conv_taps_reversed": ("acc += w[d * nk + k] * sso_conv_in(x, s0, r, nl, nk, t - (nk - 1) + k);",
                           "acc += w[d * nk + (nk - 1 - k)] * sso_conv_in(x, s0, r, nl, nk, t - (nk - 1) + k);"),
    "conv_window_offset": ("return s0 ? s0[r * (nk - 1) + (tt + nk - 1)] : 0.0;",
                           "return s0 ? s0[r * (nk - 1) + (-tt - 1)] : 0.0;"),
    "conv_bias_dropped": ("    double acc = bias ? bias[d] : 0.0;\n    for (int64_t k = 0; k < nk; k++)\n        acc += w[d * nk + k] * sso_conv_in",
                          "    double acc = 0.0;\n    for (int64_t k = 0; k < nk; k++)\n        acc += w[d * nk + k] * sso_conv_in"),
    "conv_silu_derivative_wrong": ("g *= s * (1.0 + pre * (1.0 - s));", "g *= s;"),
    "conv_dx_wrong_tap": ("dx[r * nl + tt] += w[d * nk + k] * g;", "dx[r * nl + tt] += w[d * nk + (nk - 1 - k)] * g;"),
    "conv_dwindow_dropped": ("ds0[r * (nk - 1) + (tt + nk - 1)] += w[d * nk + k] * g;",
                             "ds0[r * (nk - 1) + (tt + nk - 1)] += 0.0 * g;"),
    "conv_update_shift_wrong": ("state[r * (nk - 1) + j] = (j + 1 < nk - 1) ? state[r * (nk - 1) + j + 1] : x[r];",
                                "state[r * (nk - 1) + j] = (j > 0) ? state[r * (nk - 1) + j - 1] : x[r];"),
    "ssd_decay_sign_flipped": ("const double decay = exp(dt * A[h]);",
                               "const double decay = exp(-dt * A[h]);"),
    "ssd_input_without_dt": ("*hv = decay * *hv + dt * xt[p] * bt[n];",
                             "*hv = decay * *hv + xt[p] * bt[n];"),
    "ssd_output_uses_B": ("acc += ct[n] * *hv;", "acc += bt[n] * *hv;"),
    "ssd_group_map_wrong": ("const int64_t g = h / (nh / ng);\n            for (int64_t i = 0; i < np * ns; i++)\n                H[i]",
                            "const int64_t g = h % ng;\n            for (int64_t i = 0; i < np * ns; i++)\n                H[i]"),
    "ssd_skip_dropped": ("yt[p] = acc + (D ? D[h] * xt[p] : 0.0);", "yt[p] = acc;"),
    "ssd_h0_ignored": ("H[i] = h0 ? h0[(b * nh + h) * np * ns + i] : 0.0;", "H[i] = 0.0;"),
    "ssd_bwd_carry_missing": ("for (int64_t i = 0; i < ps; i++) Gs[i] *= a;   /* carried to t - 1 */",
                              "for (int64_t i = 0; i < ps; i++) Gs[i] *= 1.0;"),
    "ssd_bwd_dB_without_dt": ("dbt[n] += dt * *gv * xt[p];", "dbt[n] += *gv * xt[p];"),
    "ssd_bwd_dA_without_decay": ("dA[h] += dt * a * d_a;", "dA[h] += dt * d_a;"),
    "ssd_bwd_dC_previous_state": ("dct[n] += Ht[p * ns + n] * dyt[p];", "dct[n] += Hp[p * ns + n] * dyt[p];"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    with tempfile.TemporaryDirectory() as tmp:
        c = os.path.join(tmp, "mutant.c")
        so = os.path.join(tmp, "mutant.so")
        with open(c, "w") as f:
            f.write(src.replace(old, new))
        subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-o", so, c, "-lm"],
                       check=True)
        env = dict(os.environ, SS_ORACLE_LIB_OVERRIDE=so)
        res = subprocess.run(
            [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
             os.path.join(ROOT, "tests", "test_oracle_pins.py"),
             os.path.join(ROOT, "tests", "test_oracle_bwd_pins.py"),
             os.path.join(ROOT, "tests", "test_oracle_conv_pins.py"),
             os.path.join(ROOT, "tests", "test_oracle_ssd_pins.py")],
            cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
        assert res.returncode != 0, f"pins did not catch mutation {name}:\n{res.stdout[-2000:]}"
