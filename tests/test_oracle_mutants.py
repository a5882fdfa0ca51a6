"""The oracle's pins must catch plausible mistakes.  Each case plants one
mistake in a copy of the oracle's C source (on the CPU, in a temporary
directory), builds it, and expects at least one pin to fail on it.  Every
mutation keeps all memory accesses in bounds."""
import functools
import os

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "gdn_oracle.c")

MUTANTS = {
    "no_decay": ("S[e] *= gamma;", "S[e] *= 1.0;"),
    "delta_sign": ("u[c] = beta * (vt[c] - r);", "u[c] = beta * (r - vt[c]);"),
    "no_beta": ("u[c] = beta * (vt[c] - r);", "u[c] = (vt[c] - r);"),
    "khead_modulo": ("const int j = h / G;", "const int j = h % Hk;"),
    "output_uses_key": ("o += S[(size_t)kk * V + c] * qh[kk];",
                        "o += S[(size_t)kk * V + c] * kh[kk];"),
    "update_uses_query": ("S[(size_t)kk * V + c] += kh[kk] * u[c];",
                          "S[(size_t)kk * V + c] += qh[kk] * u[c];"),
    "eps_outside_root": ("double f = c / sqrt(ss + eps);",
                         "double f = c / (sqrt(ss) + eps);"),
    "no_query_scale": ("scale > 0.0 ? scale : 1.0 / sqrt((double)K)",
                       "scale > 0.0 ? scale : 1.0"),
    "softplus_drops_one": ("log1p(exp(-fabs(x)))", "log(exp(-fabs(x)) + 1e-3)"),
    "gate_not_exponentiated": ("-exp(A_log[h]) * oracle_softplus(x)",
                               "-A_log[h] * oracle_softplus(x)"),
    "gamma_half_exponent": ("const double gamma = exp(g);",
                            "const double gamma = exp(0.5 * g);"),
    "sigmoid_sign": ("return 1.0 / (1.0 + exp(-x));", "return 1.0 / (1.0 + exp(x));"),
    "dt_bias_dropped": ("a[t * Hv + h] + dt_bias[h]", "a[t * Hv + h]"),
    "no_writeback": ("                    tile_put(tile, kk * row_stride + c * col_stride, S[(size_t)kk * V + c], bf16);",
                     "                    (void)0;"),
    "layout_ignored_on_load": ("S[(size_t)kk * V + c] = tile_get(tile, kk * row_stride + c * col_stride, bf16);",
                               "S[(size_t)kk * V + c] = tile_get(tile, (size_t)kk * V + c, bf16);"),
    "bf16_truncates": ("y = ldexp(nearbyint(ldexp(m, 8)), e - 8);", "y = ldexp(trunc(ldexp(m, 8)), e - 8);"),
    "bf16_one_bit_short": ("y = ldexp(nearbyint(ldexp(m, 8)), e - 8);", "y = ldexp(nearbyint(ldexp(m, 7)), e - 7);"),
    "bf16_ties_away": ("y = ldexp(nearbyint(ldexp(m, 8)), e - 8);", "y = ldexp(round(ldexp(m, 8)), e - 8);"),
    "bf16_subnormal_as_normal": ("if (ax < 0x1p-126) {", "if (0) {"),
    "bf16_subnormal_quantum": ("y = nearbyint(x * 0x1p133) * 0x1p-133;",
                               "y = nearbyint(x * 0x1p132) * 0x1p-132;"),
    "bf16_via_float": ("const double m = frexp(x, &e);", "const double m = frexp((double)(float)x, &e);"),
    "bf16_overflow_saturates": ("const float f = (float)y;",
                                "const float f = (float)fmax(fmin(y, 0x1.fep127), -0x1.fep127);"),
    "gating_head_index": ("g[e] = -exp(A_log[h]) * oracle_softplus(a[e] + dt_bias[h]);",
                          "g[e] = -exp(A_log[0]) * oracle_softplus(a[e] + dt_bias[h]);"),
    "gating_beta_from_a": ("beta[e] = oracle_sigmoid(b[e]);", "beta[e] = oracle_sigmoid(a[e]);"),
    "intermediate_row": ("intermediate + ((size_t)t * Hv + h)",
                         "intermediate + ((size_t)(t1 - 1) * Hv + h)"),
    "varlen_end": ("cu_seqlens ? cu_seqlens[i + 1]", "cu_seqlens ? cu_seqlens[i] + 1"),
    "output_pre_update": (
        "            /* rank-1 update S += khat u^T */\n"
        "            for (int kk = 0; kk < K; ++kk)\n"
        "                for (int c = 0; c < V; ++c)\n"
        "                    S[(size_t)kk * V + c] += kh[kk] * u[c];\n"
        "            /* output o = S^T qhat */\n"
        "            double *ot = out + (t * Hv + h) * (int64_t)V;\n"
        "            for (int c = 0; c < V; ++c) {\n"
        "                double o = 0.0;\n"
        "                for (int kk = 0; kk < K; ++kk)\n"
        "                    o += S[(size_t)kk * V + c] * qh[kk];\n"
        "                ot[c] = o;\n"
        "            }\n",
        "            double *ot = out + (t * Hv + h) * (int64_t)V;\n"
        "            for (int c = 0; c < V; ++c) {\n"
        "                double o = 0.0;\n"
        "                for (int kk = 0; kk < K; ++kk)\n"
        "                    o += S[(size_t)kk * V + c] * qh[kk];\n"
        "                ot[c] = o;\n"
        "            }\n"
        "            for (int kk = 0; kk < K; ++kk)\n"
        "                for (int c = 0; c < V; ++c)\n"
        "                    S[(size_t)kk * V + c] += kh[kk] * u[c];\n"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mut = tmp_path / f"mut_{name}.c"
    mut.write_text(src.replace(old, new))
    lib = oracle.build(src=str(mut), out=str(tmp_path / f"libmut_{name}.so"))
    upd = functools.partial(oracle.update, lib_path=lib)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(upd)
        except (AssertionError, ValueError) as e:
            caught.append(f"{pin.__name__}: {str(e).splitlines()[0][:80]}")
    assert caught, f"no pin caught the planted mistake '{name}'"
