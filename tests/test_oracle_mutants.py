"""Planted mistakes in the oracle: each must fail at least one pin.

Every case copies the oracle's C source, plants one plausible mistake (a dropped
term, a wrong sign or index, a swapped operand, a wrong rounding), builds it into
a temporary library and runs the pins against it. This shows the pins would
catch such a mistake in the oracle itself. Everything here runs on the CPU.
"""
import os
import subprocess
import tempfile

import pytest

import oracle
from tests import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "lmoe_oracle.c")

MUTANTS = [
    ("ties_to_higher_index", "if (best < 0 || route_score(l[e]) > route_score(l[best]))",
     "if (best < 0 || route_score(l[e]) >= route_score(l[best]))"),
    ("nan_kept_as_nan", "return isnan(v) ? -INFINITY : (double)v;", "return (double)v;"),
    ("nan_ranked_as_plus_inf", "return isnan(v) ? -INFINITY : (double)v;", "return isnan(v) ? INFINITY : (double)v;"),
    ("infinite_max_plain_softmax", "    if (isinf(m)) {", "    if (0) {"),
    ("softmax_over_all_logits", "for (int j = 0; j < k; ++j) den += exp(route_score(l[id[j]]) - m);",
     "for (int q = 0; q < E; ++q) den += exp(route_score(l[q]) - m);"),
    ("router_bias_dropped", "if (bias) s += (double)bias[e];", ""),
    ("pooled_norm_dropped", "double r = 1.0 / sqrt(ss / Dp + eps);\n    for (int c = 0; c < Dp; ++c) p[c] = p[c] * r",
     "double r = 1.0;\n    for (int c = 0; c < Dp; ++c) p[c] = p[c] * r"),
    ("pooled_gamma_dropped", "p[c] = p[c] * r * (double)gp[c];", "p[c] = p[c] * r;"),
    ("expert_norm_dropped", "  double r = 1.0 / sqrt(ss / Dp + eps);\n  double su = 0;",
     "  double r = 1.0;\n  double su = 0;"),
    ("expert_eps_outside_sqrt", "  double r = 1.0 / sqrt(ss / Dp + eps);\n  double su = 0;",
     "  double r = 1.0 / (sqrt(ss / Dp) + eps);\n  double su = 0;"),
    ("expert_mean_over_F", "  double r = 1.0 / sqrt(ss / Dp + eps);\n  double su = 0;",
     "  double r = 1.0 / sqrt(ss / F + eps);\n  double su = 0;"),
    ("expert_gamma_dropped", "z[c] = n * (double)ge[c];", "z[c] = n;"),
    ("gate_up_swapped", "load_row(wgu, sgu, wdt, (size_t)f, Dp, row);\n    for (int c = 0; c < Dp; ++c) g +=",
     "load_row(wgu, sgu, wdt, (size_t)(F + f), Dp, row);\n    for (int c = 0; c < Dp; ++c) g +="),
    ("silu_sign", "h[f] = g / (1.0 + exp(-g)) * u;", "h[f] = g / (1.0 + exp(g)) * u;"),
    ("silu_on_up", "h[f] = g / (1.0 + exp(-g)) * u;", "h[f] = u / (1.0 + exp(-u)) * g;"),
    ("routing_weight_dropped", "acc[c] += w[(size_t)t * k + j] * z[((size_t)t * k + j) * Dp + c];",
     "acc[c] += z[((size_t)t * k + j) * Dp + c];"),
    ("norm_after_combine", "    for (int o = 0; o < D; ++o) {\n      double s = 0;",
     "    { double q = 0; for (int c = 0; c < Dp; ++c) q += acc[c] * acc[c];\n"
     "      for (int c = 0; c < Dp; ++c) acc[c] /= sqrt(q / Dp + 1e-6); }\n"
     "    for (int o = 0; o < D; ++o) {\n      double s = 0;"),
    ("unpool_transposed", "s += acc[c] * ld(wun, dt, (size_t)o * Dp + c);",
     "s += acc[c] * ld(wun, dt, (size_t)c * D + o);"),
    ("permutation_unstable", "    for (int t = 0; t < T; ++t)\n      for (int j = 0; j < k; ++j)\n        if (ids",
     "    for (int t = T - 1; t >= 0; --t)\n      for (int j = 0; j < k; ++j)\n        if (ids"),
    ("offsets_inclusive", "    offsets[e] = pos;\n    counts[e] = 0;",
     "    counts[e] = 0;"),
    ("sum_rounding_dropped", "    if (rnd)\n      for (int c = 0; c < Dp; ++c) acc[c] = orc_round_bf16(acc[c]);", ""),
    ("expert_output_rounding_dropped", "    if (rnd) y = orc_round_bf16(y);", ""),
    ("bf16_truncates", "return nearbyint(v / step) * step;\n}", "return trunc(v / step) * step;\n}"),
    ("mx_e2m1_emax", "int X = mx_block_exponent(v + 32 * b, 32, 2);", "int X = mx_block_exponent(v + 32 * b, 32, 1);"),
    ("mx_no_subnormals", "if (e < emin) e = emin;", ""),
    ("mx_e4m3_saturation", "round_minifloat(fabs(v[i]) / s, 3, -6, 448.0)", "round_minifloat(fabs(v[i]) / s, 3, -6, 480.0)"),
    ("mx_swiglu_quant_dropped", "  if (mx_act) orc_mx_quant_e4m3(h, F, NULL, NULL, h);\n  else if (rnd)",
     "  if (0) orc_mx_quant_e4m3(h, F, NULL, NULL, h);\n  else if (rnd && !mx_act)"),
    ("mxfp4_nibble_order", "uint8_t c = (i % 2 == 0) ? (row[i / 2] & 0xF) : (row[i / 2] >> 4);",
     "uint8_t c = (i % 2 == 1) ? (row[i / 2] & 0xF) : (row[i / 2] >> 4);"),
    ("nvfp4_nibble_order", "const uint8_t c = (k % 2 == 0) ? (byte & 0xF) : (byte >> 4);",
     "const uint8_t c = (k % 2 == 1) ? (byte & 0xF) : (byte >> 4);"),
    ("nvfp4_scale_per_32", "scales16[row * (cols / 16) + k / 16]", "scales16[row * (cols / 16) + k / 32]"),
    ("nvfp4_product_in_double", "v[i] = (double)x;",
     "v[i] = orc_e2m1_value(c) * orc_e4m3_value(sc) * (double)gm;"),
    ("nvfp4_matrix_scale_dropped", "const float x = p * gm;", "const float x = p;"),
    ("nvfp4_host_flush_mode_kept", "_mm_setcsr(csr & ~0x8040u);                 /* FTZ", "_mm_setcsr(csr);                 /* FTZ"),
    ("nvfp4_sign_bit_kept", "& 0x7F;\n          if (sc == 0x7F) bad = 1;", ";\n          if ((sc & 0x7F) == 0x7F) bad = 1;"),
]


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(source, name, old, new):
    assert source.count(old) == 1, f"mutation site for {name} not found exactly once"
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "lmoe_oracle.c")
        with open(path, "w") as f:
            f.write(source.replace(old, new))
        so = os.path.join(d, f"liboracle_{name}.so")
        subprocess.run(["gcc", "-O2", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared", path,
                        "-o", so, "-lm"], check=True)
        O = oracle.Oracle(so)
        caught = []
        for pin in pins.PINS:
            try:
                pin(O)
            except AssertionError:
                caught.append(pin.__name__)
        assert caught, f"no pin catches the planted mistake {name}"
