"""Plant plausible mistakes in the oracle source (on the CPU) and check that at
least one pin catches each. This is what makes the pins trustworthy: an oracle
with a dropped term, a wrong sign, a wrong index or a transposed operand does
not pass them."""
import os

import pytest

import oracle
from oracle_pins import ALL_PINS

MUTATIONS = {
    "dropped_D": ("acc + D * (double)xt[p]", "acc"),
    "sign_of_A": ("const double a = exp(d * A);", "const double a = exp(-d * A);"),
    "no_decay": ("row[n] = a * row[n] + dx * (double)Bt[n];", "row[n] = row[n] + dx * (double)Bt[n];"),
    "no_dt_on_input": ("const double dx = wi * (double)xt[p];\n            double acc = 0.0;\n            for (int n = 0; n < N; ++n) {\n                row[n] = a * row[n]",
                       "const double dx = (double)xt[p];\n            double acc = 0.0;\n            for (int n = 0; n < N; ++n) {\n                row[n] = a * row[n]"),
    "B_C_swapped": ("acc += (double)Ct[n] * row[n];\n            }\n            if (yu)", "acc += (double)Bt[n] * row[n];\n            }\n            if (yu)"),
    "output_before_update": ("row[n] = a * row[n] + dx * (double)Bt[n];\n                acc += (double)Ct[n] * row[n];",
                             "acc += (double)Ct[n] * row[n];\n                row[n] = a * row[n] + dx * (double)Bt[n];"),
    "group_index": ("const int g = h / (H / G);\n    const double A", "const int g = h % G;\n    const double A"),
    "transposed_state_read": ("acc += (double)Ct[n] * row[n];\n            }\n            if (yu)",
                              "acc += (double)Ct[n] * hs[(size_t)(n % P) * N + (p % N)];\n            }\n            if (yu)"),
    "init_ignored": ("for (size_t k = 0; k < PN; ++k) hs[k] = s0[k];", "(void)s0; memset(hs, 0, PN * sizeof(double));"),
    "bias_head_index": ("v += (double)o->dt_bias[h];", "v += (double)o->dt_bias[0];"),
    "bias_after_softplus": ("    if (o->dt_bias) v += (double)o->dt_bias[h];\n    if (o->dt_softplus) v = fmax(v, 0.0) + log1p(exp(-fabs(v)));",
                            "    if (o->dt_softplus) v = fmax(v, 0.0) + log1p(exp(-fabs(v)));\n    if (o->dt_bias) v += (double)o->dt_bias[h];"),
    "softplus_dropped_linear_part": ("v = fmax(v, 0.0) + log1p(exp(-fabs(v)));", "v = log1p(exp(-fabs(v)));"),
    "softplus_as_exp": ("v = fmax(v, 0.0) + log1p(exp(-fabs(v)));", "v = exp(v);"),
    "clamp_before_softplus": ("    if (o->dt_softplus) v = fmax(v, 0.0) + log1p(exp(-fabs(v))); /* log(1 + e^v), no overflow */\n    if (o->dt_clamp) v = fmin(fmax(v, o->dt_min), o->dt_max);",
                              "    if (o->dt_clamp) v = fmin(fmax(v, o->dt_min), o->dt_max);\n    if (o->dt_softplus) v = fmax(v, 0.0) + log1p(exp(-fabs(v)));"),
    "clamp_bounds_swapped": ("v = fmin(fmax(v, o->dt_min), o->dt_max);", "v = fmin(fmax(v, o->dt_max), o->dt_min);"),
    "zoh_as_euler": ("if (o && o->zoh) return A != 0.0 ? expm1(d * A) / A : d;", "if (o && o->zoh) return d;"),
    "zoh_sign": ("return A != 0.0 ? expm1(d * A) / A : d;", "return A != 0.0 ? -expm1(d * A) / A : d;"),
    "zoh_without_division": ("return A != 0.0 ? expm1(d * A) / A : d;", "return A != 0.0 ? expm1(d * A) : d;"),
    "zoh_times_dt": ("return A != 0.0 ? expm1(d * A) / A : d;", "return A != 0.0 ? d * expm1(d * A) / A : d;"),
    "zoh_exp_not_expm1": ("return A != 0.0 ? expm1(d * A) / A : d;", "return A != 0.0 ? exp(d * A) / A : d;"),
    "step_ignores_dt_options": ("step_size(j->opts, j->dt[bh], h)", "(double)j->dt[bh]"),
    "step_euler_weight": ("input_weight(j->opts, d, (double)j->A[h])", "d"),
    "varlen_no_reset": ("if (k > 0 && j->cu[k] == t) memset(hs, 0, PN * sizeof(double));", "if (0) {}"),
    "varlen_reset_late": ("if (k > 0 && j->cu[k] == t) memset", "if (k > 0 && j->cu[k] == t - 1) memset"),
    "varlen_capture_early": ("if (j->cu && t == j->cu[k + 1] - 1)", "if (j->cu && t == j->cu[k + 1] - 2)"),
    "varlen_wrong_slot": ("memcpy(j->seq_states + ((size_t)u * j->nseq + k) * PN",
                          "memcpy(j->seq_states + ((size_t)u * j->nseq + (k + 1) % j->nseq) * PN"),
    "varlen_boundary_off_by_one": ("while (k + 1 < j->nseq && j->cu[k + 1] <= t) ++k;",
                                   "while (k + 1 < j->nseq && j->cu[k + 1] < t) ++k;"),
    "bwd_adjoint_not_decayed": ("for (size_t k = 0; k < PN; ++k) gs[k] *= a;", "(void)a;"),
    "bwd_dinit_not_decayed_by_first_token": ("for (size_t k = 0; k < PN; ++k) gs[k] *= a;",
                                             "if (t > 0) for (size_t k = 0; k < PN; ++k) gs[k] *= a;"),
    "bwd_output_adjoint_uses_B": ("gs[(size_t)p * N + n] += (double)dyt[p] * (double)Ct[n];",
                                  "gs[(size_t)p * N + n] += (double)dyt[p] * (double)Bt[n];"),
    "bwd_dx_without_weight": ("dxt[p] = wi * gB + D * (double)dyt[p];", "dxt[p] = gB + D * (double)dyt[p];"),
    "bwd_dB_uses_dy": ("dBt[n] += wi * gr[n] * (double)xt[p];", "dBt[n] += wi * gr[n] * (double)dyt[p];"),
    "bwd_dC_from_previous_state": ("dCt[n] += (double)dyt[p] * hcur[(size_t)p * N + n];",
                                   "dCt[n] += (double)dyt[p] * hprev[(size_t)p * N + n];"),
    "bwd_dstep_sign": ("const double dstep = A * a * gh + wd * gx;", "const double dstep = -A * a * gh + wd * gx;"),
    "bwd_dA_without_weight_term": ("dA += d * a * gh + wA * gx;", "dA += d * a * gh;"),
    "bwd_softplus_slope": ("slope = 1.0 / (1.0 + exp(-v));", "slope = 1.0 / (1.0 + exp(v));"),
    "bwd_clamp_slope_inverted": ("if (o->dt_clamp && (v < o->dt_min || v > o->dt_max)) slope = 0.0;",
                                 "if (o->dt_clamp && (v >= o->dt_min && v <= o->dt_max)) slope = 0.0;"),
    "bwd_zoh_slope": ("*wd = exp(z);", "*wd = 1.0;"),
    "bwd_zoh_small_z_slope_zero": ("if (fabs(z) < 1e-3) *wA = d * d * (0.5 + z / 3.0 + z * z / 8.0);",
                                   "if (fabs(z) < 1e-3) *wA = 0.0;"),
    "bwd_zoh_small_z_linear_term": ("0.5 + z / 3.0", "0.5 + z / 6.0"),
    "bwd_zoh_small_z_leading_term": ("0.5 + z / 3.0", "0.25 + z / 3.0"),
    "bwd_dD_without_x": ("dD += (double)dyt[p] * (double)xt[p];", "dD += (double)dyt[p];"),
    "previous_token_dt_for_decay": ("const double a = exp(d * A);", "const double a = exp((t ? (double)j->dt[(tok - 1) * H + h] : d) * A);"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    before, after = MUTATIONS[name]
    src = open(oracle.SRC_PATH).read()
    # the first occurrence is in the forward recurrence (the step follows it)
    assert before in src, f"mutation anchor for {name} not present"
    mut_src = tmp_path / "mut.c"
    mut_src.write_text(src.replace(before, after, 1))
    lib = oracle.build(force=True, src=str(mut_src), out=str(tmp_path / f"libmut_{name}.so"))
    caught = []
    for pin in ALL_PINS:
        try:
            pin(lib=lib)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin caught planted mistake {name}"


def test_unmutated_source_passes_all_pins(tmp_path):
    lib = oracle.build(force=True, out=str(tmp_path / "libclean.so"))
    for pin in ALL_PINS:
        pin(lib=lib)
    assert os.path.exists(lib)
