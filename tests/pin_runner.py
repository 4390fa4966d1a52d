"""Runs the oracle pins against a given build of the oracle source.

Used by test_oracle_mutations.py in a child process: exit status 0 means
every pin passed, 1 means at least one pin failed (a crash also counts as
caught)."""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
sys.path.insert(0, os.path.dirname(HERE))

import oracle  # noqa: E402
import test_oracle_fp8 as F  # noqa: E402
import test_oracle_multi_token as Q  # noqa: E402
import test_oracle_pins as T  # noqa: E402

CHECKS = [
    T.test_block_table_example_token_placement,
    T.test_slot_mapping_example,
    T.test_decode_slot_mapping_uses_last_position,
    T.test_key_address_example,
    T.test_value_address_layout,
    lambda: T.test_oracle_matches_library_sdpa_on_contiguous_copy(1, {}),
    lambda: T.test_oracle_matches_library_sdpa_on_contiguous_copy(3, dict(S=5, len_lo=16, len_hi=90)),
    T.test_oracle_matches_pure_python_brute_force,
    T.test_single_token_returns_its_value_exactly,
    T.test_zero_query_averages_values,
    lambda: T.test_partition_merge_equals_direct(48),
    lambda: T.test_append_writes_slots_bit_exactly_and_nothing_else(1, {}),
    T.test_decode_step_reads_the_appended_token,
    F.test_decode_matches_the_library_for_every_code,
    F.test_encode_matches_the_library_on_ties_and_grids,
    F.test_saturation_beyond_the_range,
    lambda: F.test_fp8_attention_matches_library_sdpa(16, 4),
    F.test_fp8_append_places_codes_of_each_token,
    Q.test_multi_token_slot_mapping_places_rows_at_the_end,
    lambda: Q.test_matches_library_causal_attention(1, dict(q_lens=[5, 16, 1, 50])),
    lambda: Q.test_matches_library_causal_attention(3, dict(S=5, len_lo=16, len_hi=90, q_lens=4)),
    Q.test_first_row_of_a_full_prefill_returns_the_first_value,
]


def main(path):
    failed = []
    with oracle.use_library(path):
        for i, c in enumerate(CHECKS):
            try:
                c()
            except Exception as e:  # any failure counts as caught
                failed.append((i, type(e).__name__))
    print("failed checks:", failed)
    return 1 if failed else 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1]))
