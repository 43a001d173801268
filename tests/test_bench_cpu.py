"""Host-side logic of bench.py: argument handling and the step plan that the
timed region replays (no GPU needed)."""
import pytest

import bench


@pytest.mark.parametrize("steps,warmup", [(20, 5), (1, 0), (64, 64), (130, 7), (6400, 640)])
def test_any_positive_step_count_is_timed_exactly(steps, warmup):
    a = bench.resolve_steps(bench.parse(["--gpus", "1", "--steps", str(steps),
                                         "--warmup", str(warmup)]))
    assert (a.steps, a.warmup) == (steps, warmup)
    chunks = bench.step_chunks(a.steps, 0)
    assert sum(c for _, c in chunks) == steps
    assert all(1 <= c <= bench.GRAPH_LEN for _, c in chunks)
    # consecutive, in order, starting at step 0
    firsts = [f for f, _ in chunks]
    assert firsts == list(range(0, steps, bench.GRAPH_LEN))
    warm = bench.step_chunks(a.warmup, a.steps)
    assert sum(c for _, c in warm) == warmup


def test_defaults_per_workload():
    for wl, (s, w) in bench.DEFAULT_STEPS.items():
        a = bench.resolve_steps(bench.parse(["--workload", wl]))
        assert (a.steps, a.warmup) == (s, w)


@pytest.mark.parametrize("argv", [["--steps", "0"], ["--warmup", "-1"]])
def test_invalid_counts_rejected(argv):
    with pytest.raises(SystemExit):
        bench.resolve_steps(bench.parse(argv))


def test_stack_steps_are_whole_passes():
    chunks = bench.step_chunks(20, 0, size=1)
    assert chunks == [(i, 1) for i in range(20)]
