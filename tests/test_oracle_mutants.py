"""The pins must catch plausible mistakes in the oracle.

Each case plants one mistake in a copy of ``oracle/zq_oracle.c`` (on the CPU,
in a temporary directory), builds it, and runs the pin suite against it with
``ZQ_ORACLE_LIB``; the suite must fail.  The committed oracle is untouched.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "zq_oracle.c")

MUTANTS = {
    # Eq. (2) read literally: S = max|x| (codes collapse to -1, 0, 1)
    "scale_without_qmax": ("s = amax / (float)qmax;", "s = amax;"),
    # ties away from zero instead of to even
    "round_half_away": ("r = rintf(x);", "r = roundf(x);"),
    # truncation instead of rounding
    "truncate": ("r = rintf(x);", "r = truncf(x);"),
    # unbiased variance in LayerNorm
    "ln_unbiased_var": ("var /= K;", "var /= (K - 1);"),
    # eps dropped from LayerNorm
    "ln_no_eps": ("sqrt(var + (double)eps)", "sqrt(var)"),
    # wrong operand index in the GEMM
    "gemm_shifted_k": ("s += (int64_t)a[k] * (int64_t)b[k];",
                       "s += (int64_t)a[k] * (int64_t)b[(k + 1) % K];"),
    # weight scale looked up by token instead of by output group
    "epilogue_scale_by_token": ("(double)sw[n / G]", "(double)sw[t % (N / G)]"),
    # bias dropped
    "epilogue_no_bias": ("v += zqo_half_to_double(bias[n]);", "v += 0.0;"),
    # GeLU with erf(x) instead of erf(x / sqrt 2)
    "gelu_wrong_arg": ("erf(v / sqrt(2.0))", "erf(v)"),
    # W4 nibbles not sign-extended
    "w4_no_sign_extend": ("if (lo >= 8)\n                lo -= 16;", ""),
    # W4 nibble order swapped
    "w4_nibble_order": ("(uint8_t)(lo | (hi << 4))", "(uint8_t)(hi | (lo << 4))"),
    # binary16 rounding by truncation
    "half_truncates": ("n = rint(a / quantum);", "n = floor(a / quantum);"),
    # W8A16: activation index off by one
    "w8a16_shifted_k": ("s += zqo_half_to_double(a[k]) * w;",
                        "s += zqo_half_to_double(a[(k + 1) % K]) * w;"),
    # W8A16: group scale not applied
    "w8a16_no_scale": ("double w = (double)sw[n / G] * (double)b[k];",
                       "double w = (double)b[k];"),
    # W8A16: bias dropped
    "w8a16_no_bias": ("s += zqo_half_to_double(bias[n]);", "s += 0.0;"),
    # W8A16: GeLU with erf(x) instead of erf(x / sqrt 2)
    "w8a16_gelu_wrong_arg": ("erf(s / sqrt(2.0))", "erf(s)"),
    # static range: momentum applied to the batch instead of the state
    "static_momentum_swapped": ("float a1 = momentum * state[1], b1 = w * mx;",
                                "float a1 = w * state[1], b1 = momentum * mx;"),
    # static scale without qmax
    "static_scale_no_qmax": ("fabsf(state[1])) / 127.0f;", "fabsf(state[1]));"),
    # first batch not used to initialize
    "static_first_ignored": ("    if (first) {\n        state[0] = mn;",
                             "    if (0) {\n        state[0] = mn;"),
    # static range: the minimum updated with the batch maximum
    "static_min_from_max": ("b0 = w * mn;", "b0 = w * mx;"),
    # static quantization without the clamp to the calibrated range
    "static_no_clamp": ("        if (x > (float)qmax)\n            x = (float)qmax;\n"
                        "        if (x < -(float)qmax)\n            x = -(float)qmax;\n",
                        ""),
    # LayerNorm variance about zero instead of about the mean
    "ln_var_not_centred": ("double d = zqo_half_to_double(row[k]) - mean;",
                           "double d = zqo_half_to_double(row[k]);"),
    # LayerNorm output not centred
    "ln_out_not_centred": ("(zqo_half_to_double(row[k]) - mean) / denom",
                           "zqo_half_to_double(row[k]) / denom"),
    # LayerNorm weight and bias swapped
    "ln_gamma_beta_swapped": ("/ denom * g + b;", "/ denom * b + g;"),
    # scale from the signed maximum instead of max |x|
    "scale_signed_max": ("float a = fabsf((float)zqo_half_to_double(v[i]));",
                         "float a = (float)zqo_half_to_double(v[i]);"),
    # W4 code range [-8, 8] read as qmax = 8
    "w4_qmax_8": ("        qmax = 7;", "        qmax = 8;"),
    # weight group of one row instead of G rows (scale of the first row only)
    "weight_group_one_row": ("quantize_unit(w + off, (size_t)G * K, qmax, q + off)",
                             "quantize_unit(w + off, (size_t)K, qmax, q + off);"
                             " quantize_with_scale(w + off, (size_t)G * K, sw[g],"
                             " qmax, q + off)"),
    # int8 codes read as unsigned in the GEMM
    "gemm_unsigned_codes": ("s += (int64_t)a[k] * (int64_t)b[k];",
                            "s += (int64_t)(uint8_t)a[k] * (int64_t)b[k];"),
    # token scale not applied in the epilogue
    "epilogue_no_token_scale": ("(double)acc[idx] * (double)sx[t] * (double)sw[n / G]",
                                "(double)acc[idx] * (double)sw[n / G]"),
    # GeLU applied before the bias is added
    "epilogue_gelu_before_bias": (
        "        if (bias)\n            v += zqo_half_to_double(bias[n]);\n"
        "        if (act == 1)\n            v = 0.5 * v * (1.0 + erf(v / sqrt(2.0)));\n",
        "        if (act == 1)\n            v = 0.5 * v * (1.0 + erf(v / sqrt(2.0)));\n"
        "        if (bias)\n            v += zqo_half_to_double(bias[n]);\n"),
    # binary16 subnormals with quantum 2^-25
    "half_subnormal_quantum": ("v = ldexp((double)m, -24);",
                               "v = ldexp((double)m, -25);"),
    # binary16 overflow one binade late
    "half_overflow_late": ("if (ex > 15)", "if (ex > 16)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    mutated = src.replace(old, new)
    c = tmp_path / "mut.c"
    c.write_text(mutated)
    so = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-std=c99", "-O2", "-fopenmp", "-fPIC", "-shared",
                    "-o", str(so), str(c), "-lm"], check=True)
    env = dict(os.environ, ZQ_ORACLE_LIB=str(so))
    r = subprocess.run(
        [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
         os.path.join(ROOT, "tests", "test_oracle_pins.py")],
        env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, (
        f"pins did not catch mutant {name}:\n{r.stdout[-2000:]}")
