"""The oracle's pins can fire: plant one plausible mistake at a time in a copy
of the oracle's C source, compile that copy on the CPU, and require that at
least one pin rejects it.  Each mutation is a slip the pages warn about or
one that a transcription of the rules invites (a wrong shift, a wrong index,
a dropped term, a swapped nibble, a lost sign of zero)."""
import os

import pytest

import oracle
import test_oracle_pins as pins

MUTATIONS = {
    "q6_k_scale_index": ("b[192 + 8 * h + l / 16 + 2 * g]", "b[192 + 8 * h + l / 16 + g]"),
    "q4_k_nibble_halves": ("const unsigned q = (r % 64) < 32 ? (byte & 15u) : (unsigned)(byte >> 4);\n        return d * (double)sc",
                           "const unsigned q = (r % 64) < 32 ? (unsigned)(byte >> 4) : (byte & 15u);\n        return d * (double)sc"),
    "k4_scale_high_bits": ("*sc = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);", "*sc = (s[j + 4] & 15) | ((s[j] >> 6) << 4);"),
    "k4_min_dropped": ("- dmin * (double)mn;\n    }\n    case OK_Q5_K", ";\n    }\n    case OK_Q5_K"),
    "iq4_xs_scales_h_shift": ("(((scales_h >> (2 * ib)) & 3u) << 4)", "(((scales_h >> (2 * (ib & 1))) & 3u) << 4)"),
    "q3_k_hmask_inverted": ("q2 - (hbit ? 0 : 4)", "q2 - (hbit ? 4 : 0)"),
    "q3_k_scale_bias": ("((low4 | (high2 << 4)) - 32)", "((low4 | (high2 << 4)) - 31)"),
    "q5_0_qh_shift": ("(((qh >> r) & 1u) << 4)", "(((qh >> (r % 16)) & 1u) << 4)"),
    "q5_k_qh_bit": ("(((unsigned)(b[16 + r % 32] >> (r / 32)) & 1u) << 4)", "(((unsigned)(b[16 + r % 32] >> (r / 64)) & 1u) << 4)"),
    "q2_k_scale_index": ("const unsigned s = b[r / 16];", "const unsigned s = b[r / 32];"),
    "q4_0_bias": ("(int)split_nibble(b + 2, r) - 8", "(int)split_nibble(b + 2, r) - 7"),
    "interleaved_nibbles": ("return t < 16 ? (q[t] & 15u) : (unsigned)(q[t - 16] >> 4);",
                            "return (t & 1) == 0 ? (q[t / 2] & 15u) : (unsigned)(q[t / 2] >> 4);"),
    "mxfp4_negative_zero": ("    -0.0, -0.5, -1.0", "    0.0, -0.5, -1.0"),
    "iq4_table_swap": ("1, 13, 25, 38,", "1, 13, 38, 25,"),
    "e8m0_bias": ("return ldexp(1.0, (int)e - 127);", "return ldexp(1.0, (int)e - 128);"),
    "f16_subnormal": ("v = ldexp((double)f, -24);", "v = ldexp((double)f, -25);"),
    "f16_exponent_bias": ("v = ldexp((double)(1024u + f), (int)e - 25);", "v = ldexp((double)(1024u + f), (int)e - 24);"),
    "matmul_reversed_x": ("acc += w[k] * x[k];\n                    mag += fabs(w[k]) * fabs(x[k]);\n                }\n                Y[m * n_sel + i]",
                          "acc += w[k] * x[K - 1 - k];\n                    mag += fabs(w[k]) * fabs(x[k]);\n                }\n                Y[m * n_sel + i]"),
    "moe_wrong_expert": ("const int64_t e = ids[p];", "const int64_t e = ids[p] ^ 1;"),
    # The same slip in both off-page kinds (their shared code placement), so
    # that tying them to each other cannot see it; only the pins against the
    # on-page Q4_K and Q6_K can.
    "k2_k3_plane_order": ("j = (r % 128) / 32, l = r % 32;", "j = 3 - (r % 128) / 32, l = r % 32;", 2),
    "k2_k3_half_order": ("const int n = r / 128, j", "const int n = 1 - r / 128, j", 2),
}


def _all_pin_cases():
    cases = []
    for blk in pins._golden_blocks():
        cases.append((pins.test_hand_decoded_block, {"blk": blk}))
    for fn in (pins.test_binary16_exhaustive, pins.test_e8m0_every_byte, pins.test_q4_0_bias,
               pins.test_q5_0_fifth_bit_splice, pins.test_q5_k_without_high_bits_is_q4_k,
               pins.test_iq4_xs_with_unit_scales_is_iq4_nl,
               pins.test_q3_k_full_mask_is_q2_k_without_mins, pins.test_q2_k_is_q4_k_with_two_bit_codes,
               pins.test_q3_k_is_q6_k_with_three_bit_codes, pins.test_moe_matches_per_expert_matmul):
        cases.append((fn, {}))
    for kind in pins.ALL_KINDS:
        for fn in (pins.test_bit_ownership, pins.test_matmul_exact_brute_force,
                   pins.test_matmul_against_numpy_and_unit_vectors):
            cases.append((fn, {"kind": kind}))
    return cases


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_reject_planted_mistake(name, tmp_path):
    old, new, *count = MUTATIONS[name]
    with open(oracle.SOURCE) as f:
        src = f.read()
    assert src.count(old) == (count[0] if count else 1), f"mutation {name} no longer matches the oracle source"
    path = os.path.join(tmp_path, "mutant.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    mutant = oracle.Oracle(oracle.compile_library(path, os.path.join(tmp_path, "libmutant.so")))
    for fn, kwargs in _all_pin_cases():
        try:
            fn(mutant, **kwargs)
        except (AssertionError, RuntimeError):
            return
    pytest.fail(f"no pin rejects the planted mistake {name}")
