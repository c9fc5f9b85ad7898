"""Host-side rule of the placement tuning: how many candidate arenas it allocates."""

import pytest

from zero_sharded_mixed_buffer_amd.optimizer import TUNE_MAX_ARENAS, tune_arena_count

GB = 10 ** 9


@pytest.mark.parametrize("free,arena,want", [
    (270 * GB, 137 * GB, 1),     # the Llama-sized arena: one fits in half the free memory
    (270 * GB, 4.8 * GB, 28),    # the Qwen rank's arena
    (270 * GB, 18.5 * GB, 7),    # the MoE rank's arena with its all-gather input
    (270 * GB, 28 * GB, 4),      # the ragged list's arena
    (1e12, 1e6, TUNE_MAX_ARENAS),  # small arenas: the count cap binds
    (1 * GB, 2 * GB, 1),         # not even one fits in the budget: still one candidate
])
def test_candidate_count_follows_the_memory_budget(free, arena, want):
    assert tune_arena_count(free, arena) == want


def test_candidate_count_overrides_and_bad_sizes():
    assert tune_arena_count(100 * GB, 10 * GB, max_arenas=3) == 3
    assert tune_arena_count(100 * GB, 10 * GB, fraction=0.25) == 2
    assert tune_arena_count(100 * GB, 10 * GB, fraction=1.0) == 10
    with pytest.raises(ValueError):
        tune_arena_count(100 * GB, 0)
