"""The oracle pins must catch plausible mistakes.

Each case below plants one mistake in a private copy of ``oracle/oracle.c``
(a dropped term, a wrong sign, a transposed index, a wrong base, an off-by-one
shard bound ...), builds that copy with gcc into a temporary directory, swaps it
in for the real oracle, and runs the pin checks of ``test_oracle_pins``.  At
least one pin must fail for every mutant.  The real oracle is restored after
each case.  Everything here runs on the CPU; nothing is written into the tree.
"""
import ctypes
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "drop_normalisation": ("acc += (w[s] / S) * o;", "acc += w[s] * o;"),
    "wrong_sign_base_e": ("w[s] = exp(x - M);", "w[s] = exp(M - x);"),
    "wrong_base_2_weight": ("w[s] = exp2(x - M);", "w[s] = exp(x - M);"),
    "transposed_head_index": ("O[(b * H + s * h_local + j) * D + d]", "O[(b * H + j * cp + s) * D + d]"),
    "swapped_lse_log_base": ("log(S) : log2(S)", "log2(S) : log(S)"),
    "merged_lse_drops_max": ("out_lse[row] = M + (", "out_lse[row] = ("),
    "bhc_offset_transposed": ("return (b * h_local + j) * cp + s;", "return (b * cp + s) * h_local + j;"),
    "bh1_offset_transposed": ("return b * (h_local * cp) + s * h_local + j;",
                              "return b * (h_local * cp) + j * cp + s;"),
    "empty_row_lse_zero": ("if (out_lse) out_lse[row] = -INFINITY;", "if (out_lse) out_lse[row] = 0.0;"),
    "empty_row_output_nan": ("                o_row[d] = 0.0;\n                if (a_row)",
                             "                o_row[d] = NAN;\n                if (a_row)"),
    "empty_payload_read": ("if (w[s] == 0.0) continue;", ";"),
    "max_ignores_first_shard": ("for (int64_t s = 0; s < cp; ++s) {\n            double x = lse[lse_offset"
                                "(lse_layout, b, j, s, h_local, cp)];\n            if (x > M)",
                                "for (int64_t s = 1; s < cp; ++s) {\n            double x = lse[lse_offset"
                                "(lse_layout, b, j, s, h_local, cp)];\n            if (x > M)"),
    "attention_no_scale": ("        z *= scale;\n        double p", "        double p"),
    "attention_value_from_tail": ("o[d] += p * dec(k[d]);", "o[d] += p * dec(k[d + (dqk - dv)]);"),
    "attention_f16_decoded_as_bf16": ("return dtype == ORACLE_F16 ? oracle_f16_to_f64 : oracle_bf16_to_f64;",
                                      "return oracle_bf16_to_f64;"),
    "attention_lse_drops_max": ("return m + log(l);", "return log(l);"),
    "attention_base2_inverted": ("if (lse_mode == ORACLE_BASE_2) lse *= M_LOG2E;",
                                 "if (lse_mode == ORACLE_BASE_2) lse /= M_LOG2E;"),
    "shard_bound_off_by_one": ("*t1 = ((s + 1) * T) / cp;", "*t1 = ((s + 1) * T) / cp + (s == 0);"),
    "bf16_decode_shift": ("((uint32_t)bits) << 16", "((uint32_t)bits) << 15"),
    "varlen_interleave_offset": ("                t0 = s;\n                step = cp;", "                t0 = s + 1;\n                step = cp;"),
    "varlen_interleave_count": ("n = L > s ? (L - s + cp - 1) / cp : 0;", "n = L > s ? (L - s) / cp : 0;"),
    "varlen_first_token_length": ("const int64_t L = seq_lens[b];", "const int64_t L = seq_lens[0];"),
    "varlen_shared_cache_offset": ("const uint16_t* cache = kv + b * kv_sb * dqk;", "const uint16_t* cache = kv;"),
    "f16_decode_bias": ("ldexp((double)(1024 + frac), expo - 25)", "ldexp((double)(1024 + frac), expo - 24)"),
    "f16_subnormal_scale": ("v = ldexp((double)frac, -24);", "v = ldexp((double)frac, -25);"),
    "f16_merge_decodes_as_bf16": ("return merge_16bit(oracle_decode_f16,", "return merge_16bit(oracle_decode_bf16,"),
}


def _pin_checks():
    """The pin tests, with concrete parameters, as zero-argument callables."""
    E, T2 = oracle.BASE_E, oracle.BASE_2
    checks = [lambda c=c: pins.test_golden_closed_forms(c) for c in pins.GOLDEN_CASES]
    checks += [
        pins.test_all_empty_output_is_positive_zero,
        pins.test_bf16_decode_matches_torch,
        pins.test_f16_decode_matches_numpy_for_every_bit_pattern,
        pins.test_f16_entry_equals_f64_entry,
        lambda: pins.test_cp1_is_identity(E),
        lambda: pins.test_equal_lse_gives_mean(4, E),
        lambda: pins.test_equal_lse_gives_mean(8, T2),
        lambda: pins.test_common_shift_is_invariant(E),
        pins.test_base2_equals_base_e_after_conversion,
        lambda: pins.test_general_merge_matches_scipy_softmax(4, T2),
        lambda: pins.test_general_merge_matches_scipy_softmax(2, E),
        lambda: pins.test_one_hot_lse_selects_head_group(oracle.LSE_BHC),
        lambda: pins.test_one_hot_lse_selects_head_group(oracle.LSE_BH1),
        pins.test_bhc_and_bh1_layouts_agree,
        pins.test_empty_shards_equal_merge_without_them,
        pins.test_full_attention_matches_scipy,
        pins.test_f16_attention_matches_scipy,
        lambda: pins.test_varlen_partials_match_scipy(False),
        lambda: pins.test_varlen_partials_match_scipy(True),
        lambda: pins.test_varlen_merged_shards_equal_full_attention(True),
        lambda: pins.test_partials_are_softmax_over_contiguous_shards(130, 4),
        lambda: pins.test_merged_partials_equal_full_attention(256, 4, T2),
    ]
    return checks


def _build_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation %s no longer matches oracle.c" % name
    mutated = src.replace(old, new)
    c_path = tmp_path / ("%s.c" % name)
    so_path = tmp_path / ("lib%s.so" % name)
    c_path.write_text(mutated)
    subprocess.run(["gcc", "-O2", "-std=gnu11", "-fPIC", "-shared", "-fopenmp", str(c_path), "-o", str(so_path),
                    "-lm"], check=True)
    return str(so_path)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    so = _build_mutant(tmp_path, name, old, new)
    real = oracle._load()
    oracle._lib = oracle._configure(ctypes.CDLL(so))
    caught = []
    try:
        for check in _pin_checks():
            try:
                check()
            except (AssertionError, ValueError, FloatingPointError):
                caught.append(check)
                break
    finally:
        oracle._lib = real
    assert caught, "no pin caught the planted mistake %r" % name


def test_unmutated_copy_passes_every_pin(tmp_path):
    so = _build_mutant(tmp_path, "identity", "#include <math.h>", "#include <math.h>")
    real = oracle._load()
    oracle._lib = oracle._configure(ctypes.CDLL(so))
    try:
        for check in _pin_checks():
            check()
    finally:
        oracle._lib = real
