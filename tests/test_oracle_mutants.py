"""Planted mistakes in the oracle must each fail at least one pin (CPU only).

Each mutant is a copy of oracle/oracle.c with one plausible mistake (a dropped
term, a wrong sign or index, a transposed operand, a wrong composition order),
compiled with gcc into a temporary directory.  If every pin still passed for
some mutant, the pins would not be pinning that part of the oracle.
"""
import os

import pytest

import oracle
from oracle import build as obuild
import oracle_pins

MUTANTS = {
    "drop_D_skip": ("if (D) y += D[d] * x;", ""),
    "exp_sign": ("h[n] = exp(dt * A_d[n]) * h[n]", "h[n] = exp(-dt * A_d[n]) * h[n]"),
    "drop_dt_in_input": ("(input_coef(dt, A_d[n], zoh) * B_t[n]) * x", "(B_t[n]) * x"),
    "A_same_for_all_n": ("h[n] = exp(dt * A_d[n])", "h[n] = exp(dt * A_d[0])"),
    "readout_uses_B": ("y += C_t[n] * h[n]", "y += B_t[n] * h[n]"),
    "B_state_index": ("(input_coef(dt, A_d[n], zoh) * B_t[n]) * x", "(input_coef(dt, A_d[n], zoh) * B_t[N - 1 - n]) * x"),
    "gate_sigmoid": ("return z / (1.0 + exp(-z));", "return 1.0 / (1.0 + exp(-z));"),
    "softplus_drop_max": ("return fmax(u, 0.0) + log1p(exp(-fabs(u)));", "return log1p(exp(-fabs(u)));"),
    "softplus_sign": ("log1p(exp(-fabs(u)))", "log1p(exp(fabs(u)))"),
    "bias_ignored": ("double u = delta + (bias ? bias[d] : 0.0);", "double u = delta;"),
    "readout_before_update": (
        "  for (int64_t n = 0; n < N; ++n) h[n] = exp(dt * A_d[n]) * h[n] + (input_coef(dt, A_d[n], zoh) * B_t[n]) * x;\n"
        "  double y = 0.0;\n  for (int64_t n = 0; n < N; ++n) y += C_t[n] * h[n];\n",
        "  double y = 0.0;\n  for (int64_t n = 0; n < N; ++n) y += C_t[n] * h[n];\n"
        "  for (int64_t n = 0; n < N; ++n) h[n] = exp(dt * A_d[n]) * h[n] + (input_coef(dt, A_d[n], zoh) * B_t[n]) * x;\n"),
    "B_previous_step": ("const double* Bt = j->B + (b * j->L + t) * j->N;",
                        "const double* Bt = j->B + (b * j->L + (t > 0 ? t - 1 : 0)) * j->N;"),
    "x_batch_index": ("int64_t e = (b * j->L + t) * j->Dn + d;          /* [batch, L, d_inner] */",
                      "int64_t e = (t) * j->Dn + d + 0 * b;"),
    "A_transposed": ("j->A + d * j->N, Bt", "j->A + d, Bt"),
    "compose_order": ("acc_b[n] = a2 * acc_b[n] + b2;", "acc_b[n] = acc_a[n] * b2 + acc_b[n];"),
    "compose_example": ("double nb = a2[i] * b1[i] + b2[i];", "double nb = a1[i] * b2[i] + b1[i];"),
    "decode_B_row": ("A + d * N, B + b * N, C + b * N", "A + d * N, B, C + b * N"),
    "last_state_index": ("j->last_state[(b * j->Dn + d) * j->N + n] = h[n];",
                         "j->last_state[(d * j->N + n) * 0 + (b * j->Dn + d) * j->N + (j->N - 1 - n)] = h[n];"),
    "gate_before_skip": ("  if (D) y += D[d] * x;\n  if (zp) y *= silu(*zp);",
                         "  if (zp) y *= silu(*zp);\n  if (D) y += D[d] * x;"),
    "h0_ignored": ("h[n] = j->h0 ? j->h0[(b * j->Dn + d) * j->N + n] : 0.0;", "h[n] = 0.0;"),
    "h0_chunked_ignored": ("acc_b[n] = j->h0 ? j->h0[(b * j->Dn + d) * N + n] : 0.0; }",
                           "acc_b[n] = 0.0; }"),
    "conv_filter_not_reversed": ("acc += w[d * K + k] * conv_input(x, state_in, b, t - K + 1 + k, d, L, Dn, K);",
                                 "acc += w[d * K + (K - 1 - k)] * conv_input(x, state_in, b, t - K + 1 + k, d, L, Dn, K);"),
    "conv_not_causal": ("conv_input(x, state_in, b, t - K + 1 + k, d, L, Dn, K);",
                        "conv_input(x, state_in, b, t + k, d, L, Dn, K);"),
    "conv_state_off_by_one": ("return state_in ? state_in[(b * Dn + d) * K + (t + K)] : 0.0;",
                              "return state_in ? state_in[(b * Dn + d) * K + (t + K - 1 < 0 ? 0 : t + K - 1)] : 0.0;"),
    "conv_update_no_shift": ("for (int64_t k = 0; k + 1 < K; ++k) st[k] = st[k + 1];", ""),
    "conv_bias_dropped": ("double acc = bias ? bias[d] : 0.0;\n        for (int64_t k = 0; k < K; ++k)\n          acc +=",
                          "double acc = 0.0;\n        for (int64_t k = 0; k < K; ++k)\n          acc +="),
    "bwd_carry_before_input": ("dh[n] += dy * Ct[n];                                  /* dh_t */",
                               "dh[n] = dh[n] * exp(dt * A_d[n]) + dy * Ct[n];"),
    "bwd_dB_drops_dt": ("dB[(b * L + t) * N + n] += dh[n] * dt * x[e];", "dB[(b * L + t) * N + n] += dh[n] * x[e];"),
    "bwd_dC_uses_hprev": ("dC[(b * L + t) * N + n] += dy * hs[(t + 1) * N + n];",
                          "dC[(b * L + t) * N + n] += dy * hs[t * N + n];"),
    "bwd_ddt_drops_input": ("ddt += dh[n] * (A_d[n] * a * hprev + Bt[n] * x[e]);", "ddt += dh[n] * (A_d[n] * a * hprev);"),
    "bwd_dA_drops_dt": ("dA[d * N + n] += dh[n] * a * hprev * dt;", "dA[d * N + n] += dh[n] * a * hprev;"),
    "bwd_dx_drops_skip": ("dx[e] = (D ? dy * D[d] : 0.0) + dt * sB;", "dx[e] = dt * sB;"),
    "bwd_softplus_derivative": ("double dd = softplus_on ? ddt * sigmoid(u) : ddt;", "double dd = ddt;"),
    "bwd_silu_derivative": ("dz[e] = dout[e] * y * (s * (1.0 + zz * (1.0 - s)));", "dz[e] = dout[e] * y * s;"),
    "bwd_dlast_ignored": ("dh[n] = dlast ? dlast[(b * Dn + d) * N + n] : 0.0;", "dh[n] = 0.0;"),
    "zoh_ignored": ("  if (!zoh) return dt;\n  if (a == 0.0)", "  return dt;\n  if (a == 0.0)"),
    "zoh_sign": ("return expm1(dt * a) / a;", "return expm1(-dt * a) / -a;"),
    "zoh_extra_factor": ("return expm1(dt * a) / a;", "return expm1(dt * a) / a * exp(0.5 * dt * a);"),
    "zoh_limit_zero": ("if (a == 0.0) return dt;", "if (a == 0.0) return 0.0;"),
    "zoh_chunked_pass1": ("Ek[n] = a * Ek[n] + (input_coef(dt, A_d[n], j->zoh) * Bt[n]) * j->x[e];",
                          "Ek[n] = a * Ek[n] + (dt * Bt[n]) * j->x[e];"),
    "zoh_decode_ignored": ("out[e] = scan_step(state + e * N, x[e], dt, zoh,", "out[e] = scan_step(state + e * N, x[e], dt, 0,"),
    "ssd_group_index": ("const int64_t g = h / (j->H / j->G);", "const int64_t g = h % j->G;"),
    "ssd_A_of_group": ("const double a = exp(dt * j->A[h]);", "const double a = exp(dt * j->A[g]);"),
    "ssd_dt_of_channel": ("step_size(j->dt[(b * j->L + t) * j->H + h]", "step_size(j->dt[(b * j->L + t) * j->H + ch % j->H]"),
    "ssd_D_per_head": ("if (j->D) y += j->D[ch] * x;", "if (j->D) y += j->D[h] * x;"),
    "ssd_state_transposed": ("j->last_state[r * j->N + n] = s[n];",
                             "j->last_state[((r / j->P) * j->N + n) * j->P + r % j->P] = s[n];"),
    "ssd_readout_before_update": ("        s[n] = a * s[n] + (dt * Bt[n]) * x;\n        y += Ct[n] * s[n];",
                                  "        y += Ct[n] * s[n];\n        s[n] = a * s[n] + (dt * Bt[n]) * x;"),
    "ssd_h0_ignored": ("s[n] = j->h0 ? j->h0[r * j->N + n] : 0.0;", "s[n] = 0.0;"),
    "ssd_decode_group": ("      const int64_t g = h / (H / G);\n      const double d", "      const int64_t g = h % G;\n      const double d"),
    "conv_state_out_oldest_last": ("state_out[(b * Dn + d) * K + k] = conv_input(x, state_in, b, L - K + k, d, L, Dn, K);",
                                   "state_out[(b * Dn + d) * K + k] = conv_input(x, state_in, b, L - 1 - k, d, L, Dn, K);"),
}


def _run_pins(orc):
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except Exception as e:  # an assertion, a shape error or NaN: the pin caught it
            failed.append((pin.__name__, type(e).__name__))
    return failed


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(obuild.SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    path = tmp_path / f"oracle_{name}.c"
    path.write_text(src.replace(old, new))
    lib = obuild.build(src=str(path), lib=str(tmp_path / f"liboracle_{name}.so"))
    failed = _run_pins(oracle.OracleLib(lib))
    assert failed, f"mutant {name} passed every pin"


def test_unmutated_copy_passes(tmp_path):
    path = tmp_path / "oracle_copy.c"
    path.write_text(open(obuild.SRC).read())
    lib = obuild.build(src=str(path), lib=str(tmp_path / "liboracle_copy.so"))
    assert _run_pins(oracle.OracleLib(lib)) == []
