"""Host-side parts of the step-graph harness (no GPU)."""

from paged_kv_split_attn_amd.step_graphs import buckets_up_to


def test_buckets_are_powers_of_two():
    assert buckets_up_to(1) == [1]
    assert buckets_up_to(16) == [1, 2, 4, 8, 16]
    assert buckets_up_to(17) == [1, 2, 4, 8, 16, 32]
    assert buckets_up_to(64) == [1, 2, 4, 8, 16, 32, 64]
