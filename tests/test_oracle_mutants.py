"""Each plausible mistake planted in a copy of the oracle must fail at least one pin.

The mistakes are planted in the oracle's C source (on the CPU, in a temporary build); the
HIP library is never involved. A mutation whose anchor text is missing fails loudly, so the
list cannot silently go stale when the oracle is edited.
"""
import os

import pytest

import oracle
import oracle_pins

MUTANTS = {
    "nibble_order_reversed": ("(w >> (4 * (k % 8)))", "(w >> (4 * (7 - k % 8)))"),
    "wrong_group_index": ("int64_t g = k / ORACLE_GROUP;",
                          "int64_t g = (k / ORACLE_GROUP + 1) % (K / ORACLE_GROUP);"),
    "zero_not_subtracted": ("int d = oracle_code(Wq, N, k, n) - zero;",
                            "int d = oracle_code(Wq, N, k, n) - 0 * zero;"),
    "zero_sign_flipped": ("int d = oracle_code(Wq, N, k, n) - zero;",
                          "int d = zero - oracle_code(Wq, N, k, n);"),
    "zero_high_nibble_kept": ("int zero = Z[g * N + n] & 0xF;", "int zero = Z[g * N + n];"),
    "scale_from_next_column": ("oracle_f16_to_f64(S[g * N + n])",
                               "oracle_f16_to_f64(S[g * N + (n + 1) % N])"),
    "codes_mirrored_columns": ("uint32_t w = Wq[(k / 8) * N + n];",
                               "uint32_t w = Wq[(k / 8) * N + (N - 1 - n)];"),
    "activations_mirrored_k": ("oracle_bf16_to_f64(A[m * K + k])",
                               "oracle_bf16_to_f64(A[m * K + (K - 1 - k)])"),
    "f16_exponent_bias": ("e - 15 - 10", "e - 16 - 10"),
    "f16_subnormal_scale": ("ldexp((double)f, -24)", "ldexp((double)f, -25)"),
    "bf16_implicit_bit": ("(double)(128 + f)", "(double)(127 + f)"),
    "bf16_subnormal_scale": ("ldexp((double)f, -126 - 7)", "ldexp((double)f, -126 - 6)"),
    "pack_shift_reversed": ("<< (4 * j);", "<< (4 * (7 - j));"),
    "pack_mask_dropped": ("(uint32_t)(q[(8 * kb + j) * N + n] & 0xF)", "(uint32_t)(q[(8 * kb + j) * N + n])"),
    "abs_sum_signed": ("abs_acc[m] += fabs(t);", "abs_acc[m] += t;"),
    "accumulate_in_float": ("acc[m] += t;", "acc[m] = (float)(acc[m] + t);"),
    # binary16 encoder
    "f16_enc_truncates": ("double m = rint(ldexp(a, 10 - e));", "double m = floor(ldexp(a, 10 - e));"),
    "f16_enc_ties_away": ("double m = rint(ldexp(a, 10 - e));", "double m = floor(ldexp(a, 10 - e) + 0.5);"),
    "f16_enc_exponent_bias": ("(uint16_t)((e + 15) << 10)", "(uint16_t)((e + 16) << 10)"),
    "f16_enc_no_subnormals": ("double m = rint(ldexp(a, 24));", "double m = 0.0 * rint(ldexp(a, 24));"),
    # quantizer
    "quant_codes_ties_away": ("rintf(w / s) + (float)z", "roundf(w / s) + (float)z"),
    "quant_codes_floor": ("rintf(w / s) + (float)z", "floorf(w / s) + (float)z"),
    "quant_range_without_zero": ("float lo = 0.0f, hi = 0.0f;", "float lo = INFINITY, hi = -INFINITY;"),
    "quant_sixteen_steps": ("oracle_f32_to_f16((hi - lo) / 15.0f)", "oracle_f32_to_f16((hi - lo) / 16.0f)"),
    "quant_zero_sign": ("rintf(-lo / s)", "rintf(lo / s)"),
    "quant_zero_truncated": ("rintf(-lo / s)", "truncf(-lo / s)"),
    "quant_degenerate_zero": ("                z = 8;", "                z = 0;"),
    "quant_nibble_order": ("(uint32_t)q << (4 * (k % 8))", "(uint32_t)q << (4 * (7 - k % 8))"),
    "quant_scale_from_next_column": ("S[g * N + n] = sb;", "S[g * N + (n + 1) % N] = sb;"),
    # 8-bit variant
    "w8_byte_order_reversed": ("(word >> (8 * (k % 4)))", "(word >> (8 * (3 - k % 4)))"),
    "w8_code_masked_to_nibble": ("(8 * (k % 4))) & 0xFFu)", "(8 * (k % 4))) & 0xFu)"),
    "w8_zero_masked_to_nibble": ("int zp = Z[grp * N + n];", "int zp = Z[grp * N + n] & 0xF;"),
    "w8_zero_not_subtracted": ("int diff = oracle_byte_code(Wq8, N, k, n) - zp;",
                               "int diff = oracle_byte_code(Wq8, N, k, n);"),
    "w8_group_of_64": ("int64_t grp = k / ORACLE_GROUP;", "int64_t grp = k / 64 / 2 * 2 % (K / ORACLE_GROUP);"),
    "w8_group_shifted": ("int64_t grp = k / ORACLE_GROUP;", "int64_t grp = ((k + 64) / ORACLE_GROUP) % (K / ORACLE_GROUP);"),
    "w8_scale_from_next_column": ("oracle_f16_to_f64(S[grp * N + n])", "oracle_f16_to_f64(S[grp * N + (n + 1) % N])"),
    "w8_codes_mirrored_columns": ("uint32_t word = Wq8[(k / 4) * N + n];", "uint32_t word = Wq8[(k / 4) * N + (N - 1 - n)];"),
    "w8_word_row_off_by_one": ("uint32_t word = Wq8[(k / 4) * N + n];", "uint32_t word = Wq8[((k / 4) ^ 1) * N + n];"),
    "w8_abs_sum_signed": ("abs_sum[m] += fabs(term);", "abs_sum[m] += term;"),
    "w8_pack_shift_reversed": ("<< (8 * j);", "<< (8 * (3 - j));"),
    "w8_pack_nibbles": ("word |= (uint32_t)q[(4 * kb + j) * N + n] << (8 * j);",
                        "word |= (uint32_t)(q[(4 * kb + j) * N + n] & 0xF) << (8 * j);"),
    # 4-bit activations (W4A4)
    "a4_divisor_eight": ("const float sa = amax / 7.0f;", "const float sa = amax / 8.0f;"),
    "a4_amax_signed": ("amax = fmaxf(amax, fabsf((float)oracle_bf16_to_f64(A[m * K + k])));",
                       "amax = fmaxf(amax, (float)oracle_bf16_to_f64(A[m * K + k]));"),
    "a4_ties_away": ("fmaxf(rintf(a / sa), -8.0f)", "fmaxf(roundf(a / sa), -8.0f)"),
    "a4_truncate": ("fmaxf(rintf(a / sa), -8.0f)", "fmaxf(truncf(a / sa), -8.0f)"),
    "a4_offset_seven": ("(uint32_t)(qa + 8) << (4 * (k % 8))", "(uint32_t)(qa + 7) << (4 * (k % 8))"),
    "a4_decode_offset_seven": ("& 0xFu) - 8;", "& 0xFu) - 7;"),
    "a4_nibble_order": ("(Aq[m * (K / 8) + k / 8] >> (4 * (k % 8)))", "(Aq[m * (K / 8) + k / 8] >> (4 * (7 - k % 8)))"),
    "a4_scale_wrong_group": ("(double)As[m * G + gk]", "(double)As[m * G + (gk + 1) % G]"),
    "a4_scale_wrong_row": ("(double)As[m * G + gk]", "(double)As[((m + 1) % M) * G + gk]"),
    "a4_weight_zero_dropped": ("(oracle_code(Wq, N, k, n) - (Z[gk * N + n] & 0xF))", "(oracle_code(Wq, N, k, n))"),
    "a4_abs_signed": ("magnitude += fabs(term);", "magnitude += term;"),
    "a4_activation_row_swapped": ("oracle_act_code(Aq, K, m, k)", "oracle_act_code(Aq, K, (m + 1) % M, k)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    with open(oracle.SOURCE) as f:
        src = f.read()
    assert src.count(old) >= 1, f"anchor for mutant {name} not found in the oracle source"
    mutated = src.replace(old, new)
    path = tmp_path / f"{name}.c"
    path.write_text(mutated)
    lib = oracle.build(str(tmp_path / f"lib_{name}.so"), source=str(path))
    o = oracle.Oracle(lib)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(o)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
