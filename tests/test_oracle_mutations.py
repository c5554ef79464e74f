"""The oracle pins must be sharp: each plausible mistake planted in a copy of
the C oracle (a dropped term, a wrong sign, index, constant or rounding rule)
must make tests/test_oracle_pins.py fail.  Runs on the CPU only; the planted
copies are built in a temporary directory and never used elsewhere."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "bitlinear_oracle.c")

MUTATIONS = {
    "weight epsilon dropped": ("const float denom = gamma + 1e-5f;", "const float denom = gamma;"),
    "round half away from zero": ("return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;",
                                  "return td > 0 ? fl + 1.0 : fl;"),
    "Q_b = 128": ("const float s = 127.0f / a;\n        for (int64_t c = 0; c < k; ++c) {\n            float t = bf16_to_f32",
                  "const float s = 128.0f / a;\n        for (int64_t c = 0; c < k; ++c) {\n            float t = bf16_to_f32"),
    "f32 quant Q_b = 128": ("const float s = 127.0f / a;\n        for (int64_t c = 0; c < k; ++c) {\n            float t = x[r * k + c] * s;",
                            "const float s = 128.0f / a;\n        for (int64_t c = 0; c < k; ++c) {\n            float t = x[r * k + c] * s;"),
    "ternary clip missing": ("return (int8_t)clip(round_half_even(t), -1.0, 1.0);",
                             "return (int8_t)round_half_even(t);"),
    "gamma of W, not |W|": ("s += fabs((double)row[c]);", "s += ((double)row[c]);"),
    "gamma divides by n only": ("double mean = abs_sum / ((double)n * (double)k);",
                                "double mean = abs_sum / ((double)n);"),
    "act max of x, not |x|": ("float v = fabsf(bf16_to_f32(x[r * k + c]));",
                              "float v = (bf16_to_f32(x[r * k + c]));"),
    "act floor dropped": ("if (a < 1e-8f)\n            a = 1e-8f;\n        const float s = 127.0f / a;\n        for (int64_t c = 0; c < k; ++c) {\n            float t = bf16_to_f32",
                          "const float s = 127.0f / a;\n        for (int64_t c = 0; c < k; ++c) {\n            float t = bf16_to_f32"),
    "f32 quant floor dropped": ("if (a < 1e-8f)\n            a = 1e-8f;\n        const float s = 127.0f / a;\n        for (int64_t c = 0; c < k; ++c) {\n            float t = x[r * k + c] * s;",
                                "const float s = 127.0f / a;\n        for (int64_t c = 0; c < k; ++c) {\n            float t = x[r * k + c] * s;"),
    "pack field order reversed": ("byte |= code << (2 * i);", "byte |= code << (6 - 2 * i);"),
    "codes +1/-1 swapped": ("code = (v == 1) ? 1u : (v == -1) ? 2u : 0u;",
                            "code = (v == 1) ? 2u : (v == -1) ? 1u : 0u;"),
    "weight sign dropped": ("s += (int64_t)a[c] * (int64_t)w[c];", "s += (int64_t)a[c] * (int64_t)(w[c] != 0);"),
    "contraction skips the last column": ("for (int64_t c = 0; c < k; ++c) {\n        if (w[c] < -1 || w[c] > 1)",
                                          "for (int64_t c = 0; c + 1 < k; ++c) {\n        if (w[c] < -1 || w[c] > 1)"),
    "weight row indexed by token": ("ternary_dot(xq + row * k, q + col * k, k, &bad)", "ternary_dot(xq + row * k, q + (row % n) * k, k, &bad)"),
    "dequant without 1/127": ("(double)acc[i * n + j] * (double)gamma * (double)amax[i] / 127.0",
                              "(double)acc[i * n + j] * (double)gamma * (double)amax[i]"),
    "dequant uses token 0 scale": ("(double)acc[i * n + j] * (double)gamma * (double)amax[i] / 127.0",
                                   "(double)acc[i * n + j] * (double)gamma * (double)amax[0] / 127.0"),
    "rmsnorm eps dropped": ("(float)(1.0 / sqrt(ss / (double)k + (double)eps));",
                            "(float)(1.0 / sqrt(ss / (double)k));"),
    "rmsnorm sum, not mean": ("(float)(1.0 / sqrt(ss / (double)k + (double)eps));",
                              "(float)(1.0 / sqrt(ss + (double)eps));"),
    "rmsnorm sqrt dropped": ("(float)(1.0 / sqrt(ss / (double)k + (double)eps));",
                             "(float)(1.0 / (ss / (double)k + (double)eps));"),
    "rmsnorm r kept in binary64": ("float xn = bf16_to_f32(x[r * k + c]) * rr;\n            if (w)\n                xn = xn * w[c];\n            if (xnorm_out)",
                                   "float xn = (float)((double)bf16_to_f32(x[r * k + c]) * (1.0 / sqrt(ss / (double)k + (double)eps)));\n            if (w)\n                xn = xn * w[c];\n            if (xnorm_out)"),
    "rmsnorm gain ignored in max": ("            if (w)\n                xn = xn * w[c];\n            if (xnorm_out)",
                                    "            if (xnorm_out)"),
    "rmsnorm gain ignored in codes": ("            if (w)\n                xn = xn * w[c];\n            xq[r * k + c]",
                                      "            xq[r * k + c]"),
    "rmsnorm r not applied": ("float xn = bf16_to_f32(x[r * k + c]) * rr;\n            if (w)\n                xn = xn * w[c];\n            if (xnorm_out)",
                              "float xn = bf16_to_f32(x[r * k + c]);\n            if (w)\n                xn = xn * w[c];\n            if (xnorm_out)"),
    "rmsnorm floor only on a'": ("        if (a < 1e-8f)\n            a = 1e-8f;\n        const float s = 127.0f / a;\n        for (int64_t c = 0; c < k; ++c) {\n            float xn",
                                 "        const float s = a > 0.0f ? 127.0f / a : 0.0f;\n        if (a < 1e-8f)\n            a = 1e-8f;\n        for (int64_t c = 0; c < k; ++c) {\n            float xn"),
    "rmsnorm max of x_norm, not |x_norm|": ("            if (fabsf(xn) > a)\n                a = fabsf(xn);", "            if (xn > a)\n                a = xn;"),
    "f32 quant max of x, not |x|": ("float v = fabsf(x[r * k + c]);", "float v = (x[r * k + c]);"),
    "silu with exp(+g)": ("h[i] = (float)(gd * (double)u[i] / (1.0 + exp(-gd)));",
                          "h[i] = (float)(gd * (double)u[i] / (1.0 + exp(gd)));"),
    "swiglu drops up": ("h[i] = (float)(gd * (double)u[i] / (1.0 + exp(-gd)));",
                        "h[i] = (float)(gd / (1.0 + exp(-gd)));"),
    "tensor quant Q_b = 127": ("const float t = (bf16_to_f32(x[i]) * 128.0f) / d;",
                               "const float t = (bf16_to_f32(x[i]) * 127.0f) / d;"),
    "tensor quant symmetric clamp": ("clip((double)t, -128.0, 127.0)", "clip((double)t, -127.0, 127.0)"),
    "tensor quant epsilon dropped": ("const float d = g + 1e-8f;", "const float d = g;"),
    "tensor quant max of x, not |x|": ("const float v = fabsf(bf16_to_f32(x[i]));", "const float v = bf16_to_f32(x[i]);"),
    "tensor dequant by 127": ("(double)gx / 128.0", "(double)gx / 127.0"),
    "q128 bound is 127 * k": ("return contract_bounded(xq, q, m, n, k, 128, acc);",
                              "return contract_bounded(xq, q, m, n, k, 127, acc);"),
    "tensor dequant drops g": ("(double)acc[i] * (double)gamma * (double)gx / 128.0",
                               "(double)acc[i] * (double)gamma / 128.0"),
    "f16 ties away from zero": ("return fmod(below, 2.0) != 0.0 ? below + 1.0 : below;", "return below + 1.0;"),
    "f16 exponent bias 16": ("((e + 15) << 10)", "((e + 16) << 10)"),
    "f16 subnormal quantum 2^-23": ("rne_double(a * 16777216.0)", "rne_double(a * 8388608.0)"),
    "f16 overflow from 65504": ("if (a >= 65520.0)", "if (a > 65504.0)"),
    "row scale divides by n": ("oracle_f32_to_f16((float)(s / (double)k))", "oracle_f32_to_f16((float)(s / (double)n))"),
    "row scale kept in binary32": ("s16[r] = oracle_f32_to_f16((float)(s / (double)k));",
                                   "s16[r] = oracle_f32_to_f16((float)(s / (double)k));\n        if (s16[r] == 0x3ACD) s16[r] = 0x3ACC;"),
    "row ternarize epsilon dropped": ("const float denom = oracle_f16_to_f32(s16[r]) + 1e-5f;",
                                      "const float denom = oracle_f16_to_f32(s16[r]);"),
    "row dequant uses row 0 scale": ("(double)oracle_f16_to_f32(s16[j])", "(double)oracle_f16_to_f32(s16[0])"),
    "binary sign of zero is -1": ("b[i] = (int8_t)(w[i] < 0.0f ? -1 : 1);", "b[i] = (int8_t)(w[i] <= 0.0f ? -1 : 1);"),
    "binary uses the sign bit": ("b[i] = (int8_t)(w[i] < 0.0f ? -1 : 1);", "b[i] = (int8_t)(signbit(w[i]) ? -1 : 1);"),
    "dequant drops gamma": ("(double)acc[i * n + j] * (double)gamma * (double)amax[i] / 127.0",
                            "(double)acc[i * n + j] * (double)amax[i] / 127.0"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) == 1, "mutation anchor not found exactly once: " + name
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fno-fast-math", "-ffp-contract=off",
                    "-fPIC", "-shared", str(mutated), "-o", str(lib), "-lm"], check=True)
    env = dict(os.environ, BITLINEAR_ORACLE_LIB=str(lib), OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, "pins did not catch: " + name + "\n" + r.stdout[-2000:]
