"""moe_residency_plan (host logic of the C ABI) against the oracle's plan,
without a GPU: the plan touches no device memory."""
import os

import numpy as np
import pytest

import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "bit_quantized_expert_router_amd", "libmoe_q2.so")
pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")


def _random_occupants(rng, E, S):
    cur = np.full(S, -1, dtype=np.int32)
    held = rng.choice(E, size=rng.integers(0, S + 1), replace=False)
    cur[rng.choice(S, size=held.size, replace=False)] = held
    return cur


@pytest.mark.parametrize("seed", range(6))
def test_plan_matches_oracle(seed):
    from bit_quantized_expert_router_amd import binding as B
    rng = np.random.default_rng(seed)
    for _ in range(40):
        E = int(rng.integers(1, 80))
        S = int(rng.integers(0, E + 1))
        # few distinct values, so equal counts are common
        counts = rng.integers(0, 6, size=E).astype(np.uint64)
        cur = _random_occupants(rng, E, S)
        new, slot_of, n = B.moe_residency_plan(counts, S, cur)
        r_new, r_slot_of, r_changed = O.residency_plan(counts, S, cur)
        np.testing.assert_array_equal(new, r_new)
        np.testing.assert_array_equal(slot_of, r_slot_of)
        assert n == r_changed.size


def test_plan_large_counts_and_full_size():
    """E = 1024, counts beyond 2^32 (uint64 all the way)."""
    from bit_quantized_expert_router_amd import binding as B
    rng = np.random.default_rng(7)
    E, S = 1024, 700
    counts = (rng.integers(0, 4, size=E).astype(np.uint64) << np.uint64(33)) + rng.integers(0, 3, size=E).astype(np.uint64)
    cur = _random_occupants(rng, E, S)
    new, slot_of, n = B.moe_residency_plan(counts, S, cur)
    r_new, r_slot_of, r_changed = O.residency_plan(counts, S, cur)
    np.testing.assert_array_equal(new, r_new)
    np.testing.assert_array_equal(slot_of, r_slot_of)
    assert n == r_changed.size


def test_plan_rejects_bad_occupants():
    from bit_quantized_expert_router_amd import binding as B
    counts = np.arange(8, dtype=np.uint64)
    for cur in ([1, 1, -1], [8, -1, -1], [-2, 0, 1]):
        with pytest.raises(B.MoeError):
            B.moe_residency_plan(counts, 3, cur)
    with pytest.raises(B.MoeError):
        B.moe_residency_plan(counts, 9, [-1] * 9)
