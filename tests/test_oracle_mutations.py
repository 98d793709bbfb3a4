"""Plant plausible mistakes in copies of the oracle source; the pins must catch each.

Every mutation is compiled from a modified copy of the oracle's C source into a
temporary directory (CPU only); the real oracle is untouched.
"""
import os

import pytest

from oracle_pins import PINS

MUTATIONS = {
    # name: list of (original text, replacement)
    "drop_beta_term": [("const double old = (double)beta * (double)C0[at];",
                        "const double old = 0.0;")],
    "sign_of_beta_term": [("return use_product ? alpha * acc + old : old;",
                           "return use_product ? alpha * acc - old : old;")],
    "beta_zero_adds_plus_zero": [("return use_product ? alpha * acc : 0.0;",
                                  "return use_product ? alpha * acc + 0.0 : 0.0;")],
    "no_product_adds_plus_zero": [("return use_product ? alpha * acc + old : old;",
                                   "return use_product ? alpha * acc + old : 0.0 + old;")],
    "ignore_alpha": [("combine(use_product, a_s, acc[j], beta, C0,",
                      "combine(use_product, 1.0, acc[j], beta, C0,")],
    "drop_last_k": [("for (int k = 0; k < K; ++k) {\n                    const double a",
                     "for (int k = 0; k < K - 1; ++k) {\n                    const double a")],
    "reversed_k_in_A": [("const double a = (double)A[(long)i * lda + k];",
                         "const double a = (double)A[(long)i * lda + (K - 1 - k)];")],
    "float_accumulation": [("acc[j] += p;", "acc[j] = (float)(acc[j] + p);")],
    "signed_magnitude": [("aac[j] += fabs(p);", "aac[j] += p;")],
    "beta_one_ignored_when_alpha_zero": [("const int use_product = (alpha != 0.0f) && (K > 0);\n    const double a_s",
                                          "const int use_product = 1;\n    const double a_s")],
    "op_transposed_reading_swapped": [("return (double)(trans ? X[c * ld + r] : X[r * ld + c]);",
                                       "return (double)(trans ? X[r * ld + c] : X[c * ld + r]);")],
    "op_B_indices_swapped": [("op_elem(B, ldb, trans_b, k, j)", "op_elem(B, ldb, trans_b, j, k)")],
    "op_A_uses_ldb": [("op_elem(A, lda, trans_a, i, k)", "op_elem(A, ldb, trans_a, i, k)")],
    "op_ignores_trans_b": [("op_elem(B, ldb, trans_b, k, j)", "op_elem(B, ldb, 0, k, j)")],
    "op_drop_first_k": [("for (int k = 0; k < K; ++k) {\n        const double p = op_elem",
                         "for (int k = 1; k < K; ++k) {\n        const double p = op_elem")],
    "op_entries_beta_dropped": [("op_dot(trans_a, trans_b, K, A, lda, B, ldb, i, j, &acc, &aac);\n"
                                 "        out[t] = combine(use_product, (double)alpha, acc, beta, C0,",
                                 "op_dot(trans_a, trans_b, K, A, lda, B, ldb, i, j, &acc, &aac);\n"
                                 "        out[t] = combine(use_product, (double)alpha, acc, 0.0f, C0,")],
    "op_full_alpha_ignored": [("Cref[(long)i * N + j] = combine(use_product, (double)alpha, acc, beta, C0,",
                               "Cref[(long)i * N + j] = combine(use_product, 1.0, acc, beta, C0,")],
    "bf16_bias_126": [("decode_16(in[t], 8, 7, 127)", "decode_16(in[t], 8, 7, 126)")],
    "f16_no_subnormals": [("x = ldexp((double)f / scale, 1 - bias);", "x = 0.0;")],
    "subnormal_exponent_off_by_one": [("x = ldexp((double)f / scale, 1 - bias);", "x = ldexp((double)f / scale, -bias);")],
    "implicit_one_dropped": [("x = ldexp(1.0 + (double)f / scale, (int)e - bias);", "x = ldexp((double)f / scale, (int)e - bias);")],
    "sign_ignored": [("return (float)(sign ? -x : x);", "return (float)x;")],
    "f16_fraction_bits_9": [("decode_16(in[t], 5, 10, 15)", "decode_16(in[t], 5, 9, 15)")],
    "row_stride_of_A_is_K": [("const double a = (double)A[(long)i * lda + k];",
                              "const double a = (double)A[(long)i * K + k];")],
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(oracle_mod, tmp_path, name):
    src = open(oracle_mod.SOURCE_PATH).read()
    for old, new in MUTATIONS[name]:
        assert src.count(old) == 1, f"mutation {name} does not apply to exactly one place"
        src = src.replace(old, new)
    path = tmp_path / f"mut_{name}.c"
    path.write_text(src)
    lib = oracle_mod.compile_source(str(path), str(tmp_path / f"lib_{name}.so"))
    mutant = oracle_mod.BoundOracle(lib)
    caught = []
    for pin in PINS:
        try:
            pin(mutant)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutation {name}"
