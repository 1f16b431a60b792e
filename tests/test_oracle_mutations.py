"""The pins must catch plausible mistakes in the oracle.

Each case copies the oracle's C source to a temporary directory, plants one
mistake (a dropped term, a wrong index or sign, a transposed operand, a
different reading of a step), builds it with gcc and runs the CPU pins
against it.  At least one pin must fail for every mutant.  Nothing here
touches a GPU or the HIP path.
"""
import pathlib

import numpy as np
import pytest

from oracle import Oracle, build
from oracle.engram_oracle import SOURCE
from tests import test_oracle_hash as H
from tests import test_oracle_lookup as L
from tests import test_oracle_conv as CV
from tests import test_oracle_signsgd as G
from tests import test_oracle_slice as SL

MUTANTS = {
    "drop_current_token": ("for (int k = 0; k < g; ++k)", "for (int k = 1; k < g; ++k)"),
    "every_order_full_window": ("for (int k = 0; k < g; ++k)",
                                "for (int k = 0; k < ngram_size; ++k)"),
    "reset_at_eos_not_after": ("if (tok[j] == eos_id)", "if (tok[j + 1] == eos_id)"),
    "ignore_segments": ("if (seg != NULL && seg[j] != seg[j + 1])", "if (0)"),
    "truncating_remainder": ("        r += p;", "        r = r;"),
    "head_major_layout": ("const int64_t h = (int64_t)(g - 2) * heads_per_ngram + j;",
                          "const int64_t h = (int64_t)j * (ngram_size - 1) + (g - 2);"),
    "first_offset_only": ("offsets[h] + positive_remainder", "offsets[0] + positive_remainder"),
    "window_off_by_one": ("return tok[t - shift];", "return tok[t - shift + 1];"),
    "fill_minus_one": ("#define ORACLE_FILL 0", "#define ORACLE_FILL (-1)"),
    "xor_mix": ("mix = wrapping_add(mix, wrapping_mul(window[k], multipliers[k]));",
                "mix = mix ^ wrapping_mul(window[k], multipliers[k]);"),
    "multiplier_reversed": ("wrapping_mul(window[k], multipliers[k])",
                            "wrapping_mul(window[k], multipliers[g - 1 - k])"),
    "prime_of_first_head": ("positive_remainder(mix, primes[h])",
                            "positive_remainder(mix, primes[(g - 2) * heads_per_ngram])"),
    "gather_counts_padding": ("            if (r != -1)\n                ++bad;",
                              "            ++bad;"),
    "gather_reversed_row": ("dst[e] = src[e];", "dst[e] = src[dim - 1 - e];"),
    "fp32_accumulation": ("acc[e] += (double)bf16_bits_to_float(g[e]);",
                          "acc[e] = (float)((float)acc[e] + bf16_bits_to_float(g[e]));"),
    "overwrite_not_add": ("dst[e] = dst[e] + s;", "dst[e] = s;"),
    "no_grouping": ("if (q == 0 || refs[q].row != refs[q - 1].row)", "if (1)"),
    "sgd_ascent": ("const float updated = w - step;", "const float updated = w + step;"),
    "sgd_truncating_bf16": ("u += 0x7fffu + keep_odd;", "u += 0u * keep_odd;"),
    "sgd_ties_away": ("u += 0x7fffu + keep_odd;", "u += 0x8000u + 0u * keep_odd;"),
    "sgd_sign_of_zero_is_one": ("g < 0.0f ? -1.0f : 0.0f", "g < 0.0f ? -1.0f : 1.0f"),
    "conv_taps_reversed": ("weight[c * kernel_size + k]",
                           "weight[c * kernel_size + (kernel_size - 1 - k)]"),
    "conv_dilation_off_by_one": ("(int64_t)(kernel_size - 1 - k) * dilation;",
                                 "(int64_t)(kernel_size - 1 - k) * (dilation + 1);"),
    "conv_ignores_segments": ("if (seg[j] != seg[j + 1])\n                            inside = 0;",
                              "if (0)\n                            inside = 0;"),
    "conv_drops_bias": ("float acc = bias ? bf16_bits_to_float(bias[c]) : 0.0f;",
                        "float acc = 0.0f;"),
    "conv_ignores_halo": ("? bf16_bits_to_float(halo[(b * halo_len + p) * channels + c])",
                          "? 0.0f"),
    "conv_not_causal": ("const int64_t p = pos - (int64_t)(kernel_size - 1 - k) * dilation;",
                        "const int64_t p = pos - (int64_t)(kernel_size - 1 - k) * dilation + dilation;"),
}

# Every pin, called directly with the mutant in place of the oracle fixture.
PINS = [
    lambda o: [H.test_unit_multiplier_exposes_window(o, c) for c in H.WINDOW_CASES],
    lambda o: H.test_current_token_multiplier(o),
    lambda o: H.test_exhaustive_small_alphabet(o, 3, 2, 6, 7),
    lambda o: H.test_exhaustive_small_alphabet(o, 4, 2, 6, 7),
    lambda o: H.test_exhaustive_with_segments(o, 3, 2),
    lambda o: [H.test_wraparound_edge_values(o, s) for s in range(3)],
    lambda o: H.test_zero_multipliers_give_offsets(o),
    lambda o: H.test_rows_stay_in_head_range(o),
    lambda o: H.test_heads_grouped_by_order(o),
    lambda o: L.test_gather_matches_fancy_indexing(o, 32),
    lambda o: L.test_gather_padding_and_invalid_rows(o),
    lambda o: L.test_dense_matches_add_at(o, 64, 2000, 8),
    lambda o: L.test_dense_distinct_rows_is_plain_add(o),
    lambda o: L.test_dense_one_shared_row(o),
    lambda o: L.test_dense_skips_padding_and_counts_invalid(o),
    lambda o: L.test_rowsparse_matches_dense(o),
    lambda o: [G.test_matches_torch_rounding(o, lr) for lr in (2.0 ** -8, 0.3)],
    lambda o: G.test_hand_cases_and_ties(o),
    lambda o: G.test_unlisted_rows_and_invalid_ids(o),
    lambda o: [SL.test_slice_reads_history_across_the_boundary(o, c) for c in SL.SLICE_CASES],
    lambda o: CV.test_matches_conv1d_on_exact_data(o, 4, 3, True),
    lambda o: CV.test_segments_match_one_conv1d_per_segment(o),
    lambda o: CV.test_impulse_response_spans_nine_positions(o),
    lambda o: CV.test_halo_equals_joined_row(o, True),
    lambda o: CV.test_rounding_ties_to_even(o),
]


def test_every_mutation_applies():
    src = SOURCE.read_text()
    for name, (old, _) in MUTANTS.items():
        assert src.count(old) >= 1, name


def test_unmutated_source_passes_all_pins(tmp_path):
    lib = build(SOURCE, tmp_path / "liboracle_clean.so")
    o = Oracle(lib)
    for pin in PINS:
        pin(o)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    src = SOURCE.read_text().replace(old, new)
    path = pathlib.Path(tmp_path) / f"mutant_{name}.c"
    path.write_text(src)
    lib = build(path, pathlib.Path(tmp_path) / f"libmutant_{name}.so",
                extra_flags=("-Wno-unused-parameter", "-Wno-self-assign"))
    o = Oracle(lib)
    caught = []
    for i, pin in enumerate(PINS):
        try:
            with np.errstate(all="ignore"):
                pin(o)
        except (AssertionError, ValueError):
            caught.append(i)
            break
    assert caught, f"no pin caught mutant {name}"
