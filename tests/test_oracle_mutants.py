"""Planted-mistake test for the oracle's pins.

Each case copies oracle.c, plants one plausible mistake by a text
substitution (a dropped term, a wrong sign or index, a transposed operand,
a reversed order, an unstable pass), builds the copy with gcc on the CPU and
runs every pin against it. Every planted mistake must make at least one pin
fail; otherwise the pins would not be able to tell the oracle from a wrong
one.
"""
import os

import pytest

import oracle_pins
from oracle import oracle as oracle_mod

MUTANTS = [
    ("router drops the bias", "if (bias) s += (double)bias[e];", ""),
    ("router reads W_r transposed", "(double)Wr[i * E + e]", "(double)Wr[e * d + i]"),
    ("router accumulates in fp32", "double s = 0.0;\n            for (int64_t i = 0; i < d; ++i)",
     "float s = 0.0f;\n            for (int64_t i = 0; i < d; ++i)"),
    ("router rounds each product to fp32", "s += (double)X[t * ldx + i] * (double)Wr[i * E + e];",
     "s += (double)(X[t * ldx + i] * Wr[i * E + e]);"),
    ("router rounds the dot product before the bias",
     "if (bias) s += (double)bias[e];\n            L[t * E + e] = (float)s;",
     "L[t * E + e] = (float)s;\n            if (bias) L[t * E + e] += bias[e];"),
    ("router skips the last hidden index", "for (int64_t i = 0; i < d; ++i)\n                s +=",
     "for (int64_t i = 0; i + 1 < d; ++i)\n                s +="),
    ("router subtracts the bias", "if (bias) s += (double)bias[e];", "if (bias) s -= (double)bias[e];"),
    ("top-k ties go to the higher id", "l[e] > l[best]", "l[e] >= l[best]"),
    ("renormalisation inverted", "renorm ? (sel > 0.0 ? a / sel : 0.0) : a", "renorm ? a : (sel > 0.0 ? a / sel : 0.0)"),
    ("NaN logits not read as -infinity", "isnan(L[t * E + e]) ? -INFINITY : L[t * E + e]", "L[t * E + e]"),
    ("softmax denominator skips the last expert",
     "for (int64_t e = 0; e < E; ++e) {\n            p[e] = exp",
     "for (int64_t e = 0; e < E; ++e) {\n            if (e == E - 1) { p[e] = 0.0; continue; }\n            p[e] = exp"),
    ("shared weight not one", "alpha[t * kp + k + s2] = 1.0;", "alpha[t * kp + k + s2] = 0.5;"),
    ("shared id off by one", "idx[t * kp + k + s2] = (int32_t)(E + s2);",
     "idx[t * kp + k + s2] = (int32_t)(E + s2 - 1);"),
    ("offsets not a running sum", "offset[s + 1] = offset[s] + count[s];",
     "offset[s + 1] = count[s];"),
    ("cursor pass in descending route order",
     "for (int64_t i = i0; i < i1; ++i) {\n        int32_t psi = phi[idx[i]];\n        if (psi < 0) {",
     "for (int64_t i = i1 - 1; i >= i0; --i) {\n        int32_t psi = phi[idx[i]];\n        if (psi < 0) {"),
    ("record stores the rank, not the token", "rec_token[p] = (int32_t)(i / kp);",
     "rec_token[p] = (int32_t)(i % kp);"),
    ("absent routes not marked", "route_pos[i] = -1;\n            continue;", "continue;"),
    ("gate and up swapped", "h[n] = silu(g[n]) * u[n];", "h[n] = silu(u[n]) * g[n];"),
    ("SiLU dropped", "h[n] = silu(g[n]) * u[n];", "h[n] = g[n] * u[n];"),
    ("sigmoid sign flipped", "return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    ("W_down read transposed", "(double)wd[m * f + n]", "(double)wd[n * d + m]"),
    ("residual dropped", "y[m] = A ? (double)A[t * d + m] : 0.0;", "y[m] = 0.0;"),
    ("route weight not applied", "y[m] += alpha[i] * o;", "y[m] += o;"),
    ("last route of each token dropped",
     "for (int64_t j = 0; j < kp; ++j) {\n            const int64_t i = t * kp + j;",
     "for (int64_t j = 0; j < kp - 1; ++j) {\n            const int64_t i = t * kp + j;"),
    ("route mask ignored", "if (route_mask && !route_mask[i]) continue;", ""),
    ("up projection reads the gate weights", "su += (double)wu[n * d + c]", "su += (double)wg[n * d + c]"),
    ("fp8 exponent bias off by one", "v = ldexp(1.0 + (double)m / 8.0, e - 7);",
     "v = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    ("fp8 subnormals one binade low", "v = ldexp((double)m / 8.0, -6);", "v = ldexp((double)m / 8.0, -7);"),
    ("fp8 sign ignored", "out[i] = (float)(sgn ? -v : v);", "out[i] = (float)v;"),
    ("up projection takes the gate scales", "const double scu = Su ? (double)Su[e * f + n] : 1.0;",
     "const double scu = Sg ? (double)Sg[e * f + n] : 1.0;"),
    ("fp4 nibbles in the wrong order", "(k % 2 == 0) ? (byte & 15) : (byte >> 4)",
     "(k % 2 == 0) ? (byte >> 4) : (byte & 15)"),
    ("fp4 exponent bias 0", "ldexp(1.0 + 0.5 * m, e - 1)", "ldexp(1.0 + 0.5 * m, e)"),
    ("fp4 subnormal step 1", "e == 0 ? 0.5 * m", "e == 0 ? 1.0 * m"),
    ("fp4 scale blocks of 16", "scales[n * (K / 32) + k / 32]", "scales[n * (K / 32) + k / 16 % (K / 32)]"),
    ("fp4 scale bias 128", "ldexp(sgn ? -mag : mag, sc - 127)", "ldexp(sgn ? -mag : mag, sc - 128)"),
    ("down row scale not applied", "(double)wd[m * f + n] * scd * h[n]", "(double)wd[m * f + n] * h[n]"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, old, new):
    src = open(oracle_mod.SRC).read()
    assert src.count(old) == 1, f"substitution target not unique in oracle.c: {name}"
    mutant_src = tmp_path / "oracle_mutant.c"
    mutant_src.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle_mutant.so"
    oracle_mod.build(str(mutant_src), str(lib))
    orc = oracle_mod.Oracle(str(lib))
    failed = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check(orc)
        except (AssertionError, ValueError):
            failed.append(check.__name__)
    assert failed, f"no pin catches the planted mistake: {name}"
    assert os.path.exists(lib)
