"""Pins of the streaming-FFN schedule oracle: a worked example, the
conditions that define the launch rule checked by enumerating every
partition of small arrival sequences, the threshold against a closed-form
throughput curve, and the arrival order."""
import itertools

import numpy as np
import pytest

from oracle import streamffn as S


def test_worked_example():
    rows = [100, 50, 300, 20, 10, 500]
    # 100, 150, 450 >= 200 -> launch after arrival 3; 20, 30, 530 -> launch after 6
    assert S.launch_groups(rows, 200) == [3, 6]
    # the threshold is never reached: one invocation at the final flush (synchronous)
    assert S.launch_groups(rows, 10_000) == [6]
    # theta = 0: every arrival launches at once (the per-replica Async variant)
    assert S.launch_groups(rows, 0) == [1, 2, 3, 4, 5, 6]
    # reaching theta exactly launches
    assert S.launch_groups([60, 40, 1], 100) == [2, 3]
    assert S.launch_groups([], 5) == []


def valid_partitions(rows, theta):
    """All partitions of the arrivals into consecutive groups such that a
    group launches as soon as its rows reach theta -- every group's rows
    without its last arrival stay below theta -- and every group but the
    last reaches theta (the last may be a final flush)."""
    n = len(rows)
    out = []
    for cuts in itertools.product([0, 1], repeat=n - 1):
        ends = [i + 1 for i, c in enumerate(cuts) if c] + [n]
        start, ok = 0, True
        for j, e in enumerate(ends):
            g = rows[start:e]
            if sum(g[:-1]) >= theta:
                ok = False
            if j < len(ends) - 1 and sum(g) < theta:
                ok = False
            start = e
        if ok:
            out.append(ends)
    return out


@pytest.mark.parametrize("seed", range(40))
def test_rule_is_the_unique_partition(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 9))
    rows = [int(v) for v in rng.integers(0, 50, size=n)]
    theta = int(rng.integers(0, 120))
    parts = valid_partitions(rows, theta)
    assert parts == [S.launch_groups(rows, theta)]


def test_threshold_closed_form_curve():
    # saturating throughput c / (c + c0): reaches rho * (peak over the grid)
    counts = [2 ** i for i in range(6, 16)]
    c0 = 1500.0
    tp = [c / (c + c0) for c in counts]
    peak = max(tp)
    for rho in (0.5, 0.8, 0.9, 0.95):
        want = min(c for c in counts if c / (c + c0) >= rho * peak)
        assert S.threshold(counts, tp, rho) == want
    assert S.threshold(counts, tp, 0.9) == 16384    # 16384/17884 >= 0.9 * 32768/34268
    assert S.threshold(counts, tp, 1.0) == counts[-1]
    assert S.threshold(counts, tp, 0.0) == counts[0]


def test_threshold_unsorted_and_non_monotone():
    counts = [4096, 256, 1024, 512, 2048]
    tp = [100.0, 40.0, 95.0, 91.0, 88.0]
    assert S.threshold(counts, tp, 0.9) == 512      # smallest count with tp >= 90
    assert S.threshold(counts, tp, 0.95) == 1024
    with pytest.raises(ValueError):
        S.threshold([], [], 0.9)


def test_arrival_order_ascending_load():
    assert S.arrival_order([0, 5, 8, 11, 20]) == [1, 2, 0, 3]
    assert S.arrival_order([0, 0, 7]) == [0, 1]
