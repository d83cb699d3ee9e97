"""Pins for the oracle's expert-residency functions: the usage histogram
against per-element counting, and the residency plan against brute force
over every subset on tiny cases plus its invariants (the chosen set is the
S most used with ties to lower ids; experts that stay keep their slots)."""
import itertools

import numpy as np
import pytest

import oracle as O


def test_usage_counts_by_hand():
    ids = np.array([[3, 1, 3], [0, 9, -1], [1, 1, 2]])
    c = O.usage_counts(ids, 4)
    assert list(c) == [1, 3, 1, 2]                  # 9 and -1 are outside [0, 4)
    c2 = O.usage_counts(np.array([[2, 2]]), 4, c)
    assert list(c2) == [1, 3, 3, 2]


def brute_force_set(counts, S):
    """The S-subset that maximises the summed count, then (on equal sums) is
    lexicographically smallest in sorted id order -- which is the set of the
    S largest counts with ties to lower ids."""
    E = len(counts)
    best = None
    for sub in itertools.combinations(range(E), S):
        key = (-sum(counts[e] for e in sub), sub)
        if best is None or key < best:
            best = key
    return set(best[1]) if best else set()


@pytest.mark.parametrize("seed", range(6))
def test_plan_set_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    E = 7
    counts = rng.integers(0, 4, size=E)             # many ties
    for S in range(0, E + 1):
        cur = np.full(S, -1)
        new, slot_of, changed = O.residency_plan(counts, S, cur)
        assert set(int(e) for e in new) == brute_force_set(counts, S)
        assert list(changed) == list(range(S))       # every slot was empty
        for s in range(S):
            assert slot_of[new[s]] == s
        assert np.sum(slot_of >= 0) == S


def test_plan_keeps_resident_experts_in_place():
    counts = np.array([5, 0, 9, 9, 1, 7, 2, 9])
    cur = np.array([4, 2, 6, 0])                    # slots 0..3 hold experts 4, 2, 6, 0
    new, slot_of, changed = O.residency_plan(counts, 4, cur)
    # hottest: 2, 3, 7 (9 each), then 5 (7): 2 stays in slot 1; 3, 5, 7 fill slots 0, 2, 3
    assert list(new) == [3, 2, 5, 7]
    assert list(changed) == [0, 2, 3]
    assert slot_of[2] == 1 and slot_of[4] == -1 and slot_of[0] == -1


def test_plan_all_and_none():
    counts = np.arange(5)[::-1]
    new, slot_of, changed = O.residency_plan(counts, 5, np.full(5, -1))
    assert sorted(new) == [0, 1, 2, 3, 4] and np.all(slot_of >= 0)
    new, slot_of, changed = O.residency_plan(counts, 0, np.zeros(0))
    assert new.size == 0 and np.all(slot_of == -1) and changed.size == 0
