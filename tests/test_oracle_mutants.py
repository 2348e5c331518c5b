"""Every plausible mistake planted in a copy of the oracle must fail at least one pin.

Each mutant is a (search, replace) edit of oracle/moe_oracle.c; the search text must occur exactly
once, so a mutant cannot silently stop applying when the oracle changes.  The mutated copy is
compiled on the CPU into a temporary library and checked with the same pins as the real oracle.
All mutants keep every memory access in bounds.
"""
import os
import tempfile

import pytest

import oracle
import oracle_pins

MUTANTS = {
    "nibble order swapped": ("int code = (k % 2 == 0) ? (byte & 0x0F) : (byte >> 4);",
                             "int code = (k % 2 == 0) ? (byte >> 4) : (byte & 0x0F);"),
    "scale exponent off by one": ("return ldexp(1.0, e - 127);", "return ldexp(1.0, e - 126);"),
    "sign bit dropped": ("return (code & 8) ? -mag : mag;", "return mag;"),
    "magnitudes 3 and 4 swapped": ("{0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0}", "{0.0, 0.5, 1.0, 1.5, 2.0, 4.0, 3.0, 6.0}"),
    "wrong scale block": ("return orc_mxfp4(code, srow[k / 32]);", "return orc_mxfp4(code, srow[k / 64]);"),
    "gate and up swapped in SwiGLU": ("hs[(int64_t)i * I + n] = orc_silu(g) * (u * up_scale);",
                                      "hs[(int64_t)i * I + n] = orc_silu(u * up_scale) * g;"),
    "sigmoid weights from the biased keys": ("weights[(int64_t)t * k_total + j] = routed_scale * (sc[order[j]] / sel);",
                                             "weights[(int64_t)t * k_total + j] = routed_scale * (key[order[j]] / sel);"),
    "sigmoid selection ignores the bias": ("key[e] = sc[e] + (sel_bias ? (double)sel_bias[e] : 0.0);", "key[e] = sc[e];"),
    "sigmoid scale factor dropped": ("weights[(int64_t)t * k_total + j] = routed_scale * (sc[order[j]] / sel);",
                                     "weights[(int64_t)t * k_total + j] = sc[order[j]] / sel;"),
    "sigmoid of the negated logit": ("sc[e] = 1.0 / (1.0 + exp(-acc));", "sc[e] = 1.0 / (1.0 + exp(acc));"),
    "shared weight fixed at 1": ("weights[(int64_t)t * k_total + top_k + s] = shared_weight;",
                                 "weights[(int64_t)t * k_total + top_k + s] = 1.0;"),
    "int4 zero-point nibbles swapped": ("const int zero = (g % 2 == 0) ? (zrow[g / 2] & 0x0F) : (zrow[g / 2] >> 4);",
                                        "const int zero = (g % 2 == 0) ? (zrow[g / 2] >> 4) : (zrow[g / 2] & 0x0F);"),
    "int4 zero point not subtracted": ("return (double)(code - zero) * orc_f16(sbits);", "return (double)code * orc_f16(sbits);"),
    "int4 scale bytes big-endian": ("const uint16_t sbits = (uint16_t)(srow[2 * g] | (srow[2 * g + 1] << 8));",
                                    "const uint16_t sbits = (uint16_t)(srow[2 * g + 1] | (srow[2 * g] << 8));"),
    "int4 groups of 64": ("const int g = k / 32;\n    const uint16_t", "const int g = k / 64;\n    const uint16_t"),
    "nvfp4 blocks of 32": ("orc_mx_value(ORC_MX_FP8_E4M3, srow[k / 16])", "orc_mx_value(ORC_MX_FP8_E4M3, srow[k / 32])"),
    "nvfp4 tensor scale dropped": (" * (double)p->tensor_scale[e];", ";"),
    "int4 storage without zero points": ("return (32.0 * 4.0 + 16.0 + 4.0) / 32.0;", "return (32.0 * 4.0 + 16.0) / 32.0;"),
    "attenuation not applied": ("hs[(int64_t)i * I + n] = orc_silu(g) * (u * up_scale);",
                                "hs[(int64_t)i * I + n] = orc_silu(g) * u;"),
    "attenuation applied to the gate": ("hs[(int64_t)i * I + n] = orc_silu(g) * (u * up_scale);",
                                        "hs[(int64_t)i * I + n] = orc_silu(g * up_scale) * u;"),
    "row factor not restored": ("y[(int64_t)t * H + m] = (A * F) * acc;", "y[(int64_t)t * H + m] = A * acc;"),
    "row factor rounded down": ("return ldexp(1.0, f == 0.5 ? ex - 1 : ex);", "return ldexp(1.0, ex - 1);"),
    "row factor without the floor of 1": ("double m = sum > 1.0 ? sum : 1.0;", "double m = sum > 0.0 ? sum : 1.0;"),
    "SiLU sign": ("return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    "routing weights not renormalised": ("weights[(int64_t)t * k_total + j] = p[order[j]] / sel;",
                                         "weights[(int64_t)t * k_total + j] = p[order[j]];"),
    "router bias dropped": ("L[e] = acc + (bias ? (double)bias[e] : 0.0);", "L[e] = acc;"),
    "tie-break to the highest index": ("(p[a] == p[b] && a < b)", "(p[a] == p[b] && a > b)"),
    "last hidden term dropped in router": (
        "for (int h = 0; h < H; ++h)\n        acc += act_value(x, x_fmt, (int64_t)t * H + h) * (double)w_router[(int64_t)e * H + h];\n      L[e]",
        "for (int h = 0; h < H - 1; ++h)\n        acc += act_value(x, x_fmt, (int64_t)t * H + h) * (double)w_router[(int64_t)e * H + h];\n      L[e]"),
    "last hidden term dropped in sigmoid router": (
        "for (int h = 0; h < H; ++h)\n        acc += act_value(x, x_fmt, (int64_t)t * H + h) * (double)w_router[(int64_t)e * H + h];\n      sc[e]",
        "for (int h = 0; h < H - 1; ++h)\n        acc += act_value(x, x_fmt, (int64_t)t * H + h) * (double)w_router[(int64_t)e * H + h];\n      sc[e]"),
    "shared expert id off": ("ids[(int64_t)t * k_total + top_k + s] = E + s;\n      weights[(int64_t)t * k_total + top_k + s] = 1.0;",
                             "ids[(int64_t)t * k_total + top_k + s] = E - 1 - s;\n      weights[(int64_t)t * k_total + top_k + s] = 1.0;"),
    "sigmoid shared expert id off": ("ids[(int64_t)t * k_total + top_k + s] = E + s;\n      weights[(int64_t)t * k_total + top_k + s] = shared_weight;",
                                     "ids[(int64_t)t * k_total + top_k + s] = E + 1 + s;\n      weights[(int64_t)t * k_total + top_k + s] = shared_weight;"),
    "bucket order not stable": ("int pos = offsets[b] + fill[b]++;",
                                "int pos = offsets[b + 1] - 1 - fill[b]++;"),
    "combine uses reversed weights": ("acc += weights[(int64_t)t * k_total + j] * y_slots",
                                      "acc += weights[(int64_t)t * k_total + (k_total - 1 - j)] * y_slots"),
    "down projection reads the wrong row": ("for (int n = 0; n < I; ++n) wd[n] = orc_weight(&W->down, W->fmt, e, m, n);",
                                            "for (int n = 0; n < I; ++n) wd[n] = orc_weight(&W->down, W->fmt, e, (m + 1) % H, n);"),
    "fp16 exponent bias": ("v = ldexp(1024.0 + (double)fr, ex - 25);", "v = ldexp(1024.0 + (double)fr, ex - 24);"),
    "x row of the wrong token": ("int t = slot[i] / k_total;", "int t = slot[i] % T;"),
    "E4M3 bias off by one": ("if (fmt == ORC_MX_FP8_E4M3) { e_bits = 4; m_bits = 3; bias = 7; }",
                             "if (fmt == ORC_MX_FP8_E4M3) { e_bits = 4; m_bits = 3; bias = 6; }"),
    "MX ties rounded up": ("if (d < best_d || (d == best_d && c % 2 == 0)) {", "if (d <= best_d) {"),
    "MX scale emax off": ("int orc_mx_emax(int fmt) { return fmt == ORC_MX_FP8_E4M3 ? 8 : 2; }",
                          "int orc_mx_emax(int fmt) { return fmt == ORC_MX_FP8_E4M3 ? 8 : 1; }"),
    "MX scale from ceil(log2)": ("int c = (ex - 1) - orc_mx_emax(fmt) + 127;", "int c = ex - orc_mx_emax(fmt) + 127;"),
    "MX sign dropped": ("return signbit(q) ? (best | (1 << (bits - 1))) : best;", "return best;"),
    "MX x round trip skipped": ("if (act_fmt) mx_round_trip(xs + (int64_t)i * H, H, act_fmt);", ";"),
    "MX h round trip skipped": ("for (int i = 0; i < n_rows; ++i) mx_round_trip(hs + (int64_t)i * I, I, act_fmt);",
                                "for (int i = 0; i < n_rows; ++i) (void)0;"),
    "MX block of 16": ("const double *blk = v + (int64_t)r * K + 32 * b;\n      double amax = 0.0;\n      for (int i = 0; i < 32; ++i)",
                       "const double *blk = v + (int64_t)r * K + 32 * b;\n      double amax = 0.0;\n      for (int i = 0; i < 16; ++i)"),
    "probabilities mis-normalised by 1e-7": ("for (int e = 0; e < E; ++e) p[e] /= den;",
                                               "for (int e = 0; e < E; ++e) p[e] /= den * 1.0000001;"),
}


@pytest.fixture(scope="module")
def source():
    with open(oracle.SOURCE) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(source, name, tmp_path):
    search, replace = MUTANTS[name]
    assert source.count(search) == 1, f"mutant '{name}' no longer applies"
    src = tmp_path / "moe_oracle.c"
    src.write_text(source.replace(search, replace))
    lib = tmp_path / "liboracle_mutant.so"
    oracle.build(str(src), str(lib))
    mutant = oracle.Oracle(str(lib))
    failed = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check(mutant)
        except AssertionError:
            failed.append(check.__name__)
    assert failed, f"no pin catches the planted mistake '{name}'"
