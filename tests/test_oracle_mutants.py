"""Each plausible mistake planted in a copy of the oracle must fail at least one pin.

The mutants are built on the CPU from the oracle's source text with one edit each (a
dropped term, a wrong sign or index, a transposed operand, a wrong reading of the pages),
compiled into a temporary library and run through the pins of ``oracle_pins``.
"""
import os

import pytest

import oracle
import oracle_pins

MUTANTS = {
    # conv: taps reversed (true convolution instead of the page's w_k u_{t+k})
    "conv_taps_reversed": ("z += w[c * K + k] * u[t + k];",
                           "z += w[c * K + (K - 1 - k)] * u[t + k];"),
    # conv: bias dropped
    "conv_bias_dropped": ("double z = bias ? bias[c] : 0.0;\n                for (int64_t k = 0; k < K; ++k) {",
                          "double z = 0.0;\n                for (int64_t k = 0; k < K; ++k) {"),
    # conv: final state taken from x alone and zero-padded (the page's warned-against reading)
    "conv_F_zero_padded": ("final_state[(b * C + c) * (K - 1) + r] = u[L + r];",
                           "final_state[(b * C + c) * (K - 1) + r] = (L + r >= K - 1) ? u[L + r] : 0.0;"),
    # conv: the state is treated as a different segment from token 0
    "conv_state_other_segment": ("id[j] = (seq_idx && L > 0) ? seq_idx[b * L + 0] : 0;",
                                 "id[j] = (seq_idx && L > 0) ? seq_idx[b * L + 0] - 1 : 0;"),
    # conv: seq_idx mask compares with the previous token instead of the output token
    "conv_mask_wrong_anchor": ("if (seq_idx && id[t + k] != id[t + K - 1]) continue;",
                               "if (seq_idx && id[t + k] != id[t + (K > 1 ? K - 2 : 0)]) continue;"),
    # SiLU with the wrong sign
    "silu_sign": ("return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    # update: ring history off by one slot
    "ring_off_by_one": ("h = row[floor_mod(p - j, state_len)];",
                        "h = row[floor_mod(p - j + 1, state_len)];"),
    # update: negative ring positions clamped to slot 0 instead of wrapped (floor-mod)
    "ring_no_wrap": ("h = row[floor_mod(p - j, state_len)];",
                     "h = row[(p - j) < 0 ? 0 : (p - j) % state_len];"),
    # update: stores the output y instead of the input x
    "update_stores_y": ("row[floor_mod(p + i, state_len)] = xr[i];",
                        "row[floor_mod(p + i, state_len)] = o[i];"),
    # scan: dt dropped from the decay
    "scan_decay_no_dt": ("const double a = exp(d * A[h]);\n                const double* xt = x + ((b * L + t) * H + h) * P;",
                         "const double a = exp(A[h]);\n                const double* xt = x + ((b * L + t) * H + h) * P;"),
    # scan: dt dropped from the input term
    "scan_input_no_dt": ("st[p * N + n] = a * st[p * N + n] + d * xt[p] * Bt[n];\n                        acc += Ct[n] * st[p * N + n];\n                    }\n                    y[((b * L + t) * H + h) * P + p]",
                         "st[p * N + n] = a * st[p * N + n] + xt[p] * Bt[n];\n                        acc += Ct[n] * st[p * N + n];\n                    }\n                    y[((b * L + t) * H + h) * P + p]"),
    # scan: output read before the state update (off by one step)
    "scan_output_lag": ("st[p * N + n] = a * st[p * N + n] + d * xt[p] * Bt[n];\n                        acc += Ct[n] * st[p * N + n];\n                    }\n                    y[((b * L + t) * H + h) * P + p]",
                        "acc += Ct[n] * st[p * N + n];\n                        st[p * N + n] = a * st[p * N + n] + d * xt[p] * Bt[n];\n                    }\n                    y[((b * L + t) * H + h) * P + p]"),
    # scan: B and C swapped in the read-out
    "scan_B_C_swapped": ("acc += Ct[n] * st[p * N + n];\n                    }\n                    y[((b * L + t) * H + h) * P + p]",
                         "acc += Bt[n] * st[p * N + n];\n                    }\n                    y[((b * L + t) * H + h) * P + p]"),
    # scan: wrong head -> group map
    "scan_group_map": ("const int64_t g = h / heads_per_group;\n            double* st = (double*)malloc",
                       "const int64_t g = h % G;\n            double* st = (double*)malloc"),
    # scan: initial state indexed [H][B] instead of [B][H]
    "scan_init_transposed": ("st[e] = init_state ? init_state[(b * H + h) * P * N + e] : 0.0;",
                             "st[e] = init_state ? init_state[(h * B + b) * P * N + e] : 0.0;"),
    # scan: initial state ignored
    "scan_init_ignored": ("st[e] = init_state ? init_state[(b * H + h) * P * N + e] : 0.0;",
                          "st[e] = 0.0;"),
    # scan: no reset at packed-sequence boundaries
    "scan_no_reset": ("if (seq_idx && t > 0 && seq_idx[b * L + t] != seq_idx[b * L + t - 1])",
                      "if (0)"),
    # step: slot indices ignored
    "step_ignores_indices": ("const int64_t s = indices ? (int64_t)indices[b] : b;\n            if (s < 0 || s >= n_slots) {\n                for (int64_t t = 0; t < L_new; ++t)",
                             "const int64_t s = b;\n            if (s < 0 || s >= n_slots) {\n                for (int64_t t = 0; t < L_new; ++t)"),
    # conv backward: the direct path from the final state to the last inputs dropped
    "conv_bwd_no_dF": ("dext[L + r] += dfinal[(b * C + c) * (K - 1) + r];", "(void)r;"),
    # conv backward: taps reversed in du
    "conv_bwd_taps_reversed": ("dext[t + k] += dz[t] * w[c * K + k];",
                               "dext[t + k] += dz[t] * w[c * K + (K - 1 - k)];"),
    # conv backward: SiLU's derivative left out (delta = dy)
    "conv_bwd_no_dphi": ("dphi = sg * (1.0 + zt * (1.0 - sg));", "dphi = 1.0;"),
    # conv backward: SiLU's derivative taken as sigma(z) alone
    "conv_bwd_dphi_sigma": ("dphi = sg * (1.0 + zt * (1.0 - sg));", "dphi = sg;"),
    # conv backward: the weight gradient paired with the current input instead of the tap's
    "conv_bwd_dw_wrong_input": ("dwc[k] += dz[t] * ext[t + k];", "dwc[k] += dz[t] * ext[t + K - 1];"),
    # conv backward: dS / dx split one position off
    "conv_bwd_split_off_by_one": ("dx[(b * L + t) * C + c] = orc_round(dext[K - 1 + t], dx_round);",
                                  "dx[(b * L + t) * C + c] = orc_round(dext[K - 2 + t], dx_round);"),
    # conv backward: the sequence mask ignored
    "conv_bwd_no_mask": ("if (sq && seg[t + k] != seg[t + K - 1]) continue;", "if (0) continue;"),
    # initial-state gradient: the decay applied one token late
    "scan_bwd_decay_lag": ("prod *= exp(dt[(b * L + t) * H + h] * A[h]);\n                const double* Ct = Cm + ((b * L + t) * G + g) * N;\n                const double* dyt = dy + ((b * L + t) * H + h) * P;\n                for (int64_t p = 0; p < P; ++p)\n                    for (int64_t n = 0; n < N; ++n) acc[p * N + n] += dyt[p] * prod * Ct[n];",
                           "const double* Ct = Cm + ((b * L + t) * G + g) * N;\n                const double* dyt = dy + ((b * L + t) * H + h) * P;\n                for (int64_t p = 0; p < P; ++p)\n                    for (int64_t n = 0; n < N; ++n) acc[p * N + n] += dyt[p] * prod * Ct[n];\n                prod *= exp(dt[(b * L + t) * H + h] * A[h]);"),
    # initial-state gradient: packed-sequence resets ignored
    "scan_bwd_no_reset": ("if (sq && t > 0 && sq[t] != sq[t - 1]) {", "if (0) {"),
    # initial-state gradient: the final state's gradient dropped
    "scan_bwd_no_dF": ("if (alive && dfinal) v += prod * dfinal[(b * H + h) * P * N + e];", "(void)alive;"),
    # Philox with nine rounds
    "philox_nine_rounds": ("for (int round = 0; round < 10; ++round) {",
                           "for (int round = 0; round < 9; ++round) {"),
    # Philox key schedule not advanced
    "philox_key_fixed": ("k0 += ORC_PHILOX_W0;", "k0 += 0;"),
    # Box-Muller with cosine and sine swapped
    "box_muller_swapped": ("out[0] = r * cos(two_pi * u2);\n    out[1] = r * sin(two_pi * u2);",
                           "out[0] = r * sin(two_pi * u2);\n    out[1] = r * cos(two_pi * u2);"),
    # Box-Muller radius without the factor 2
    "box_muller_radius": ("const double r = sqrt(-2.0 * log(u1));", "const double r = sqrt(-log(u1));"),
    # both elements of a pair take the cosine branch
    "noise_pair_shared": ("return z[e % 2];", "return z[0];"),
    # the last two pairs of a block reuse the first two words
    "noise_word_reused": ("const uint64_t word = w[(e % 8) / 2];",
                          "const uint64_t word = w[(e % 4) / 2];"),
    # fitted noise scaled by the variance instead of the standard deviation
    "fitted_noise_var_scale": ("mean[h] + sqrt(var[h]) * z", "mean[h] + var[h] * z"),
    # EMA weights the other way round (the common convention the page warns against)
    "stats_ema_swapped": ("mean[h] = orc_round((1.0 - beta) * m + beta * mean[h], out_round);",
                          "mean[h] = orc_round(beta * m + (1.0 - beta) * mean[h], out_round);"),
    # variance without subtracting the mean
    "stats_var_uncentred": ("const double d = fin[(b * H + h) * per + e] - m;",
                            "const double d = fin[(b * H + h) * per + e];"),
    # sample variance instead of the population variance
    "stats_var_n_minus_1": ("const double v = ss / count;", "const double v = ss / (count - 1.0);"),
    # reset decision inverted (zero with probability 1 - p)
    "reset_inverted": ("const int zero = (w[b % 4] >> 32) < threshold;",
                       "const int zero = (w[b % 4] >> 32) >= threshold;"),
    # vector decay: the decay of the neighbouring state dimension
    "vdecay_wrong_dimension": ("hs[p * N + n] = an[n] * hs[p * N + n] + u * xt[p] * Bt[n];",
                               "hs[p * N + n] = an[(n + 1) % N] * hs[p * N + n] + u * xt[p] * Bt[n];"),
    # vector decay: dt dropped from the input term
    "vdecay_input_no_dt": ("hs[p * N + n] = an[n] * hs[p * N + n] + u * xt[p] * Bt[n];",
                           "hs[p * N + n] = an[n] * hs[p * N + n] + xt[p] * Bt[n];"),
    # vector decay: the rate form without dt
    "vdecay_rate_no_dt": (": exp(u * A_vec[h * N + n]);", ": exp(A_vec[h * N + n]);"),
    # vector decay: every head reads head 0's gates
    "vdecay_gate_head_0": ("an[n] = log_decay ? exp(log_decay[((b * L + t) * H + h) * N + n])",
                           "an[n] = log_decay ? exp(log_decay[((b * L + t) * H + 0) * N + n])"),
    # vector decay: packed-sequence resets ignored
    "vdecay_no_reset": ("if (row_ids && t > 0 && row_ids[t] != row_ids[t - 1])", "if (0)"),
    # vector decay: read-out before the update
    "vdecay_readout_lag": ("hs[p * N + n] = an[n] * hs[p * N + n] + u * xt[p] * Bt[n];\n                        out += Ct[n] * hs[p * N + n];",
                           "out += Ct[n] * hs[p * N + n];\n                        hs[p * N + n] = an[n] * hs[p * N + n] + u * xt[p] * Bt[n];"),
    # bf16 rounding keeps 9 bits
    "bf16_nine_bits": ("int q = e - 8;", "int q = e - 9;"),
    # bf16 rounding truncates instead of nearest-even
    "bf16_truncates": ("double r = ldexp(nearbyint(ldexp(fabs(v), -q)), q);",
                       "double r = ldexp(floor(ldexp(fabs(v), -q)), q);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    find, repl = MUTANTS[name]
    with open(oracle._SRC) as f:
        src = f.read()
    assert src.count(find) == 1, f"mutation anchor for {name} not unique/found"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(find, repl))
    so = str(tmp_path / "libmutant.so")
    oracle.build(force=True, src=str(path), out=so)
    lib = oracle.load_library(so)
    caught = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check(lib)
        except AssertionError:
            caught.append(check.__name__)
            break
    assert caught, f"mutant {name} passed every pin"
