"""The pins must fail when a plausible mistake is planted in the oracle.

Each case copies the oracle's C source to a temporary directory, applies one
textual mutation, compiles it with gcc and runs the pin suite against that
library in a child process.  Nothing here touches a GPU.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "ssm_oracle.c")

MUTATIONS = {
    "read_before_write": (
        "      hp[n] = abar * hp[n] + bbar * x; /* write the token first ... */\n"
        "      acc += Ct[n] * hp[n];            /* ... then read the state */",
        "      acc += Ct[n] * hp[n];\n      hp[n] = abar * hp[n] + bbar * x;"),
    "dropped_skip": ("double out = acc + dskip * x;", "double out = acc;"),
    "bias_twice": ("double v = raw + bias;", "double v = raw + 2.0 * bias;"),
    "softplus_twice": ("return softplus ? oracle_softplus(v) : v;",
                       "return softplus ? oracle_softplus(oracle_softplus(v)) : v;"),
    "zoh_as_euler": ("*bbar = (a != 0.0) ? expm1(kappa) / a * b : delta * b;", "*bbar = delta * b;"),
    "euler_as_zoh": ("    *bbar = delta * b;\n  }", "    *bbar = expm1(kappa) / a * b;\n  }"),
    "combine_transposed": ("*b_out = a2 * b1 + b2;", "*b_out = a1 * b2 + b1;"),
    "A_transposed": ("j->A[c * N + n]", "j->A[(n * dim + c) % (dim * N)]"),
    "B_C_swapped": ("acc += Ct[n] * hp[n];", "acc += Bt[n] * hp[n];"),
    "gate_before_skip": ("    double out = acc + dskip * x;\n    if (j->z) {\n      const double zz = j->z[xi];\n      out *= zz * oracle_sigmoid(zz);\n    }",
                         "    double out = acc;\n    if (j->z) {\n      const double zz = j->z[xi];\n      out *= zz * oracle_sigmoid(zz);\n    }\n    out += dskip * x;"),
    "decay_sign": ("  *abar = exp(kappa);", "  *abar = exp(-kappa);"),
    "sigmoid_sign": ("if (v >= 0.0) return 1.0 / (1.0 + exp(-v));", "if (v >= 0.0) return 1.0 / (1.0 + exp(v));"),
    "step_drops_state": ("      h[n] = abar * h[n] + bbar * x;\n      acc += j->C[b * N + n] * h[n];",
                         "      h[n] = bbar * x;\n      acc += j->C[b * N + n] * h[n];"),
    "padding_off_by_one": ("    if (t >= len) { /* padding: no output, state kept */",
                           "    if (t > len) { /* padding: no output, state kept */"),
    "padding_updates_state": ("      j->y[xi] = 0.0;\n      continue;", "      j->y[xi] = 0.0;"),
    "reset_ignored": ("    if (j->reset && j->reset[b * L + t]) /* a document starts at t */",
                      "    if (0) /* a document starts at t */"),
    "reset_one_token_late": ("    if (j->reset && j->reset[b * L + t]) /* a document starts at t */",
                             "    if (j->reset && t > 0 && j->reset[b * L + t - 1])"),
    "h0_ignored": ("    hp[n] = j->h0 ? j->h0[(b * dim + c) * N + n] : 0.0;", "    hp[n] = 0.0;"),
    "conv_taps_reversed": ("for (int64_t i = 0; i < k; ++i) pre += w[c * k + i] * XT(t - i, start);",
                           "for (int64_t i = 0; i < k; ++i) pre += w[c * k + (k - 1 - i)] * XT(t - i, start);"),
    "conv_not_causal": ("for (int64_t i = 0; i < k; ++i) pre += w[c * k + i] * XT(t - i, start);",
                        "for (int64_t i = 0; i < k; ++i) pre += w[c * k + i] * XT(t - i + 1, start);"),
    "conv_window_holds_outputs": ("      if (k > 1) win[(k - 2) * dim] = xt;",
                                  "      if (k > 1) win[(k - 2) * dim] = out[b * dim + c];"),
    "conv_window_newest_first": ("          const int64_t s = len - (k - 1) + j; /* oldest first */",
                                 "          const int64_t s = len - 1 - j;"),
    "conv_reset_ignored": ("        if (reset && reset[b * L + t]) start = t;", "        (void)reset;"),
    "conv_bias_dropped": ("        double pre = bias ? bias[c] : 0.0;", "        double pre = 0.0;"),
    "bwd_no_carry": ("          g[n] = doc_start ? 0.0 : g[n] * abar; /* carry to t - 1 */",
                     "          g[n] = doc_start ? 0.0 : g[n]; /* carry to t - 1 */"),
    "bwd_carry_crosses_reset": ("          g[n] = doc_start ? 0.0 : g[n] * abar; /* carry to t - 1 */",
                                "          g[n] *= abar; /* carry to t - 1 */"),
    "bwd_reset_keeps_previous_state": ("          const double dabar = doc_start ? 0.0 : g[n] * hp[n];",
                                       "          const double dabar = g[n] * hp[n];"),
    "bwd_padding_has_gradients": ("        if (t >= len) { /* padding: zero gradients, g passes through */",
                                  "        if (t >= L) { /* padding: zero gradients, g passes through */"),
    "bwd_forward_ignores_reset": ("          const double prev = doc_start ? 0.0 : hs[t * N + n];",
                                  "          const double prev = hs[t * N + n];"),
    "bwd_softplus_derivative": ("        const double dv = softplus ? ddt * oracle_sigmoid(v) : ddt;",
                                "        const double dv = softplus ? ddt * oracle_sigmoid(-v) : ddt;"),
    "bwd_zoh_ddelta_as_euler": ("            ddt += dabar * a * abar + dbbar * abar * Bt[n];",
                                "            ddt += dabar * a * abar + dbbar * Bt[n];"),
    "bwd_dA_drops_phi_prime": ("            dA[c * N + n] += dabar * dt * abar + dbbar * Bt[n] * dt * dt * phi_prime(kap);",
                               "            dA[c * N + n] += dabar * dt * abar;"),
    "bwd_dC_uses_old_state": ("          dC[(b * L + t) * N + n] += ds * ht[n];",
                              "          dC[(b * L + t) * N + n] += ds * hp[n];"),
    "bwd_silu_derivative": ("          if (dz) dz[xi] = dy[xi] * s * sg * (1.0 + zz * (1.0 - sg));",
                            "          if (dz) dz[xi] = dy[xi] * s * sg;"),
    "bwd_phi_prime_series": ("      s += (double)j * kp / term_f;", "      s += kp / term_f;"),
    "conv_bwd_silu_derivative": ("  return s * (1.0 + v * (1.0 - s));", "  return s;"),
    "conv_bwd_taps_reversed": ("          ROUTE(t - i, start, w[c * k + i] * dpre);",
                               "          ROUTE(t - i, start, w[c * k + (k - 1 - i)] * dpre);"),
    "conv_bwd_crosses_reset": ("        if (reset && reset[b * L + t]) start = t;\n        double pre = bias ? bias[c] : 0.0;\n        for (int64_t i = 0; i < k; ++i) pre += w[c * k + i] * XT(t - i, start);\n        const double dpre",
                               "        double pre = bias ? bias[c] : 0.0;\n        for (int64_t i = 0; i < k; ++i) pre += w[c * k + i] * XT(t - i, start);\n        const double dpre"),
    "conv_bwd_window_grad_dropped": ("          ROUTE(s, start, dstate_out[(b * (k - 1) + j) * dim + c]);",
                                     "          (void)s;"),
    "conv_bwd_dw_lag": ("          dw[c * k + i] += dpre * XT(t - i, start);",
                        "          dw[c * k + i] += dpre * XT(t - i + 1, start);"),
    "ssd_wrong_head_decay": ("      const double a = A[hd];", "      const double a = A[0];"),
    "ssd_weight_missing": ("            h[n] = alpha * h[n] + w * B[(b * L + t) * N + n] * xv;",
                           "            h[n] = alpha * h[n] + B[(b * L + t) * N + n] * xv;"),
    "ssd_dt_per_channel": ("          const double dt = step_size(dt_raw[(b * L + t) * nheads + hd],",
                           "          const double dt = step_size(dt_raw[(b * L + t) * nheads + (hd + p) % nheads],"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    mutated = src.replace(old, new)
    csrc = tmp_path / "mut.c"
    lib = tmp_path / "libmut.so"
    csrc.write_text(mutated)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", str(lib), str(csrc),
                    "-lm", "-pthread"], check=True)
    env = dict(os.environ, SSM_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        os.path.join(ROOT, "tests", "test_oracle_conv_pins.py"),
                        os.path.join(ROOT, "tests", "test_oracle_conv_bwd_pins.py"),
                        os.path.join(ROOT, "tests", "test_oracle_bwd_pins.py"),
                        os.path.join(ROOT, "tests", "test_oracle_ssd_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutation {name} survived the pins:\n{r.stdout[-2000:]}"
