"""Plant plausible mistakes in copies of the oracle (on the CPU) and check
that the pins catch every one of them."""
import os

import pytest

import oracle
from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "gdr_oracle.c")

# (name, exact text in the source, replacement)
MUTANTS = [
    ("gdn_sign_of_erase", "beta * v[i] - alpha * beta * sk",
     "beta * v[i] + alpha * beta * sk"),
    ("gdn_erase_without_decay", "beta * v[i] - alpha * beta * sk",
     "beta * v[i] - beta * sk"),
    ("gdn_decay_dropped", "s[j] = alpha * s[j] + c * k[j]",
     "s[j] = s[j] + c * k[j]"),
    ("gdn_write_without_beta", "const double c = beta * v[i] - alpha",
     "const double c = v[i] - alpha"),
    ("gdn_read_with_query", "sk += s[j] * k[j]", "sk += s[j] * q[j]"),
    ("gdn_output_from_key", "oi += s[j] * q[j];\n        o[i] = oi;\n    }\n}\n\n/* Gated delta rule forward",
     "oi += s[j] * k[j];\n        o[i] = oi;\n    }\n}\n\n/* Gated delta rule forward"),
    ("gdn_token_index_shift", "alpha[bth], beta[bth], o + bth * Dv);",
     "alpha[bth], beta[t + 1 < T ? bth + H : bth], o + bth * Dv);"),
    ("gdn_transposed_state_init", "memcpy(S, s0, sizeof(double) * (size_t)(Dv * Dk));",
     "for (long i = 0; i < Dv; ++i) for (long j = 0; j < Dk; ++j) S[i * Dk + j] = (i < Dk && j < Dv) ? s0[j * Dk + i] : 0.0;"),
    ("gdn2_erase_gate_dropped", "rd += s[j] * (erase[j] * k[j])",
     "rd += s[j] * k[j]"),
    ("gdn2_write_gate_dropped", "const double c = write[i] * v[i] - rd",
     "const double c = v[i] - rd"),
    ("gdn2_read_before_decay",
     "for (long j = 0; j < Dk; ++j) s[j] *= alpha[j];      /* S' */\n        double rd = 0.0;                                     /* S'(b.k) */\n        for (long j = 0; j < Dk; ++j) rd += s[j] * (erase[j] * k[j]);",
     "double rd = 0.0;\n        for (long j = 0; j < Dk; ++j) rd += s[j] * (erase[j] * k[j]);\n        for (long j = 0; j < Dk; ++j) s[j] *= alpha[j];"),
    ("gdn2_gate_on_value_axis", "s[j] *= alpha[j];", "s[j] *= alpha[i < Dk ? i : 0];"),
    ("l2norm_sum_not_squared", "ss += xr[c] * xr[c]", "ss += fabs(xr[c])"),
    ("l2norm_eps_outside_root", "1.0 / sqrt(ss + eps)", "1.0 / (sqrt(ss) + eps)"),
    ("l2norm_row_shift", "const double *xr = x + r * d;",
     "const double *xr = x + (r + 1 < n ? r + 1 : r) * d;"),
    ("l2norm_sign_lost", "out[r * d + c] = xr[c] * inv", "out[r * d + c] = fabs(xr[c]) * inv"),
    ("l2norm_bwd_projection_dropped", "dx[r * d + j] = gr[j] / nn - xr[j] * xg / (nn * nn * nn);",
     "dx[r * d + j] = gr[j] / nn;"),
    ("l2norm_bwd_eps_outside_root", "const double nn = sqrt(ss + eps);",
     "const double nn = sqrt(ss) + eps;"),
    ("l2norm_bwd_wrong_power", "xr[j] * xg / (nn * nn * nn)", "xr[j] * xg / (nn * nn)"),
    ("gate_sum_not_mean", "sqrt(ss / (double)d + eps)", "sqrt(ss + eps)"),
    ("gate_eps_outside_root", "sqrt(ss / (double)d + eps)", "(sqrt(ss / (double)d) + eps)"),
    ("gate_sigmoid_not_silu", "const double gate = grow[c] / (1.0 + exp(-grow[c]));",
     "const double gate = 1.0 / (1.0 + exp(-grow[c]));"),
    ("gate_weight_by_row", "(w ? w[c] : 1.0)", "(w ? w[r < d ? r : 0] : 1.0)"),
    ("gate_bwd_projection_dropped", "dout[rr * d + j] = dn * r - orow[j] * on * r * r * r / (double)d;",
     "dout[rr * d + j] = dn * r;"),
    ("gate_bwd_silu_derivative_as_sigmoid",
     "dg[rr * d + i] = dyr[i] * orow[i] * r * wi * sg * (1.0 + grow[i] * (1.0 - sg));",
     "dg[rr * d + i] = dyr[i] * orow[i] * r * wi * sg;"),
    ("gate_bwd_dw_without_gate", "if (dw) dw[i] += dyr[i] * orow[i] * r * grow[i] * sg;",
     "if (dw) dw[i] += dyr[i] * orow[i] * r;"),
    ("gate_bwd_sum_not_mean", "orow[j] * on * r * r * r / (double)d", "orow[j] * on * r * r * r"),
    ("bwd_dalpha_missing_read_term", "dat += gs - be * dc * u;", "dat += gs;"),
    ("bwd_dk_missing_read_path", "x += G[i * Dk + j] * cv[i] - a * be * dcv[i] * Sp[i * Dk + j];",
     "x += G[i * Dk + j] * cv[i];"),
    ("bwd_carry_without_decay", "G[i * Dk + j] = a * G[i * Dk + j] - a * be * dcv[i] * kt[j];",
     "G[i * Dk + j] = G[i * Dk + j] - a * be * dcv[i] * kt[j];"),
    ("bwd_dq_from_old_state", "x += Sn[i * Dk + j] * dot[i];", "x += Sp[i * Dk + j] * dot[i];"),
    ("bwd2_dalpha_from_new_state", "dat[j] += dsp * Sp[i * Dk + j];", "dat[j] += dsp * Sn[i * Dk + j];"),
    ("bwd2_erase_grad_sign", "dev[j] -= dcv[i] * sprime;", "dev[j] += dcv[i] * sprime;"),
    ("bwd2_carry_without_decay", "G[i * Dk + j] = dsp * at[j];", "G[i * Dk + j] = dsp;"),
    ("bwd2_write_grad_uses_w", "dwt[i] = dc * vt[i];", "dwt[i] = dc * wt[i];"),
    ("bwd_segment_off_by_one", "memcpy(st, ck + sg * SS, sizeof(double) * SS);\n                for (long t = t0; t < t1; ++t) {",
     "memcpy(st, ck + (sg > 0 ? sg - 1 : 0) * SS, sizeof(double) * SS);\n                for (long t = t0; t < t1; ++t) {"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutated = src.replace(old, new, 1)
    cpath = tmp_path / "mutant.c"
    cpath.write_text(mutated)
    lib = oracle.build(True, str(cpath), str(tmp_path / "libmutant.so"))
    orc = oracle.OracleLib(lib)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutant {name}"
