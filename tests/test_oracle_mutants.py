"""Plant plausible mistakes in copies of the oracle (on the CPU) and require
that the pins catch every one of them.

Each mutant is oracle.c with one textual substitution: a dropped term, a
wrong sign, a wrong index, a transposed operand, a wrong constant, a missing
rounding.  The copy is compiled into a temporary directory and the pins are
run against it through ``oracle.using``.
"""
import os

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "residual add dropped": ("if (r) hv += or_load(r, act, m * K + k);", "(void)r;"),
    "rms uses sum not mean": ("inv = 1.0 / sqrt(ss / (double)K + eps);", "inv = 1.0 / sqrt(ss + eps);"),
    "eps outside sqrt": ("inv = 1.0 / sqrt(ss / (double)K + eps);", "inv = 1.0 / (sqrt(ss / (double)K) + eps);"),
    "layernorm mean sign": ("n = (h[k] - mu) * inv * or_load(gamma, act, k);",
                            "n = (h[k] + mu) * inv * or_load(gamma, act, k);"),
    "layernorm unbiased variance": ("inv = 1.0 / sqrt(vs / (double)K + eps);",
                                    "inv = 1.0 / sqrt(vs / (double)(K - 1) + eps);"),
    "beta dropped": ("if (beta) n += or_load(beta, act, k);", "(void)beta;"),
    "gamma index shifted": ("n = h[k] * inv * or_load(gamma, act, k);",
                            "n = h[k] * inv * or_load(gamma, act, (k + 1) % K);"),
    "A operand not rounded": ("if (a_out) a_out[m * K + k] = or_round((double)n32, act);",
                              "if (a_out) a_out[m * K + k] = (double)n32;"),
    "A operand from the double value": ("if (a_out) a_out[m * K + k] = or_round((double)n32, act);",
                                        "if (a_out) a_out[m * K + k] = or_round(n, act);"),
    "fp32 path mean sign": ("const float d = h32 - mu32;", "const float d = h32 + mu32;"),
    "fp32 path beta dropped": ("beta ? (float)or_load(beta, act, k) : 0.0f);", "0.0f);"),
    "fp32 path rstd dropped": ("const float t = h32 * rs32;", "const float t = h32;"),
    "fp32 statistics from the wrong root": ("const float mu32 = (float)mu, rs32 = (float)inv;",
                                           "const float mu32 = (float)mu, rs32 = (float)(inv * inv);"),
    "fp8 scale not rounded to fp32": ("if (a) a[m * K + k] = or_e4m3_value(c) * (double)s;",
                                      "if (a) a[m * K + k] = or_e4m3_value(c) * ((double)amax / 448.0);"),
    "fp8 quantised from the double rows": ("float t = (float)n[m * K + k] * inv;",
                                           "float t = (float)(n[m * K + k] * ((double)OR_E4M3_MAX / (double)amax));"),
    "weight transposed": ("s += a[m * K + k] * wr[k];", "s += a[m * K + k] * or_load(w, wdtype, k * N + j);"),
    "qkv k/v swapped": ("else if (c < nq + nkv) k[m * nkv + (c - nq)] = y;",
                        "else if (c < nq + nkv) v[m * nkv + (c - nq)] = y;"),
    "swiglu gate/up swapped": ("y = or_silu(g) * u;", "y = or_silu(u) * g;"),
    "silu sign": ("return g / (1.0 + exp(-g));", "return g / (1.0 + exp(g));"),
    "gelu cubic constant": ("0.044715 * y * y * y", "0.047715 * y * y * y"),
    "gelu half dropped": ("return 0.5 * y * (1.0 + tanh", "return y * (1.0 + tanh"),
    "bias after activation": ("if (actfn == OR_ACT_GELU_TANH) y = or_gelu_tanh(y);",
                              "if (actfn == OR_ACT_GELU_TANH) y = or_gelu_tanh(y - (bias ? or_load(bias, act, j) : 0)) + (bias ? or_load(bias, act, j) : 0);"),
    "dequant single rounding": ("double w = or_round(or_round(prod, OR_F32), OR_BF16);",
                                "double w = or_round(prod, OR_BF16);"),
    "round ties away": ("double r = nearbyint(scaled);", "double r = round(scaled);"),
    "bf16 precision off by one": ("case OR_BF16: *p = 8;", "case OR_BF16: *p = 9;"),
    "fp16 subnormal decode": ("mag = ldexp((double)man, -24);", "mag = ldexp((double)man, -25);"),
    "int4 nibble order": ("int nib = (row[k / 2] >> (4 * (int)(k % 2))) & 0xF;",
                          "int nib = (row[k / 2] >> (4 * (int)(1 - k % 2))) & 0xF;"),
    "int4 not sign-extended": ("return nib >= 8 ? nib - 16 : nib;", "return nib;"),
    "int4 one scale per row": ("s[j * G + k / OR_I4_GROUP]", "s[j * G]"),
    "int4 group of 64": ("enum { OR_I4_GROUP = 128 };", "enum { OR_I4_GROUP = 64 };"),
    "down residual dropped": ("if (residual) out[m * N + c] += or_load(residual, act, m * N + c);", "(void)residual;"),
    "down residual transposed": ("if (residual) out[m * N + c] += or_load(residual, act, m * N + c);",
                                 "if (residual) out[m * N + c] += or_load(residual, act, c * M + m);"),
    "down bias shifted": ("if (bias) out[m * N + c] += or_load(bias, act, c);",
                          "if (bias) out[m * N + c] += or_load(bias, act, (c + 1) % N);"),
    "int4 signed zero kept": ("if (w == 0.0) w = 0.0;   /* +0 (R9) */", "(void)0;"),
    "e4m3 exponent bias": ("ldexp(8.0 + m, e - 10)", "ldexp(8.0 + m, e - 11)"),
    "e4m3 subnormal step": ("ldexp((double)m, -9)", "ldexp((double)m, -10)"),
    "e4m3 ties away": ("double q = nearbyint(16.0 * f - 8.0);", "double q = round(16.0 * f - 8.0);"),
    "e4m3 no mantissa carry": ("if (q == 8.0) { q = 0.0; field += 1; }", "(void)0;"),
    "fp8 activation scale dropped": ("if (a) a[m * K + k] = or_e4m3_value(c) * (double)s;",
                                     "if (a) a[m * K + k] = or_e4m3_value(c);"),
    "fp8 activations not quantised": ("if (!rc && fp8) rc = or_quant_rows_e4m3(a, M, K, NULL, a, NULL);", "(void)0;"),
    "fp8 weight scale dropped": ("wr[k] = or_e4m3_value(((const uint8_t *)w)[j * K + k]) * (double)w_scale[j];",
                                 "wr[k] = or_e4m3_value(((const uint8_t *)w)[j * K + k]);"),
    "e2m1 exponent bias": ("ldexp(2.0 + m, e - 2)", "ldexp(2.0 + m, e - 1)"),
    "e2m1 subnormal step": ("e == 0 ? 0.5 * m", "e == 0 ? 1.0 * m"),
    "e2m1 sign dropped": ("return (code & 8) ? -v : v;", "return v;"),
    "e8m0 bias": ("ldexp(1.0, s - 127)", "ldexp(1.0, s - 128)"),
    "mxfp4 nibble order": ("(row[k >> 1] >> ((k & 1) << 2)) & 0xF", "(row[k >> 1] >> ((1 - (k & 1)) << 2)) & 0xF"),
    "mxfp4 block of 16": ("enum { OR_MX_BLOCK = 32 };", "enum { OR_MX_BLOCK = 16 };"),
    "mxfp4 one scale per row": ("s[j * G + k / OR_MX_BLOCK]", "s[j * G]"),
    "mxfp4 operand not rounded": ("const double w = or_round(prod, OR_BF16);", "const double w = prod;"),
    "fp8 down input not quantised": ("if (wdtype == OR_E4M3) or_quant_rows_e4m3(ad, M, K, NULL, ad, NULL);",
                                     "(void)0;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mut = tmp_path / "oracle_mut.c"
    mut.write_text(src.replace(old, new))
    lib = oracle.build(src=str(mut), out=str(tmp_path / "liboracle_mut.so"))
    failed = []
    with oracle.using(lib):
        for pin in oracle_pins.ALL_PINS:
            try:
                pin()
            except AssertionError:
                failed.append(pin.__name__)
    assert failed, f"no pin caught the mutant '{name}'"
