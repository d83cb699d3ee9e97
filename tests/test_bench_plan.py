"""The benchmark's per-case row plan: every index that the eager, graphed
and hooked passes of a case use must lie inside the rows the case
allocates, for the driver's settings and the extremes."""
import pytest

import bench


@pytest.mark.parametrize("steps,warmup", [(20, 5), (1, 0), (400, 40), (2, 1), (7, 3)])
def test_every_phase_index_in_range(steps, warmup):
    counts = bench.case_steps(steps)
    cases = [(steps, warmup), (counts["half"], warmup), (counts["windows"], max(4, warmup // 2))]
    for n, w in cases:
        assert n >= 1
        plan = bench.step_plan(n, w)
        rows = bench.rows_needed(n, w)
        for name, idx in plan.items():
            assert all(0 <= i < rows for i in idx), (name, n, w)
        # the timed region is exactly n steps; the warm graph precedes it on other rows
        assert len(plan["graph_timed"]) == n
        assert set(plan["graph_warm"]).isdisjoint(plan["graph_timed"])
        assert len(plan["warmup"]) == w


def test_plan_rejects_empty():
    with pytest.raises(ValueError):
        bench.step_plan(0, 5)
