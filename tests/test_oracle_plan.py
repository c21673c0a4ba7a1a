"""Pins for the oracle's layer-parallel set plan."""
import os

import pytest

from oracle.plan import default_group_plan, plan_offsets, offsets_to_sets

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "plan_L32_N4.txt")


def _read_golden():
    sets = []
    for line in open(GOLDEN):
        line = line.strip()
        if line and not line.startswith("#"):
            sets.append([int(x) for x in line.split()])
    return sets


def test_worked_example_from_pages():
    # printed example: N = 4, 32 layers
    assert default_group_plan(32, 4) == _read_golden()


@pytest.mark.parametrize("L,N", [(2, 2), (4, 2), (16, 2), (16, 4), (24, 3), (32, 4), (80, 4),
                                 (5, 7), (3, 1), (1, 3), (7, 3)])
def test_plan_is_contiguous_cover_with_singleton_ends(L, N):
    sets = default_group_plan(L, N)
    offs = plan_offsets(sets)          # raises if not a contiguous ordered cover
    assert offs[-1] == L
    assert sets[0] == [0]
    if L > 1:
        assert sets[-1] == [L - 1]
    assert all(1 <= len(s) <= N for s in sets[1:-1])
    assert offsets_to_sets(offs) == sets


def test_group_size_one_is_sequential():
    assert default_group_plan(16, 1) == [[l] for l in range(16)]


@pytest.mark.parametrize("L,N,expect", [
    (16, 2, [[0], [1], [2, 3], [4, 5], [6, 7], [8, 9], [10, 11], [12, 13], [14], [15]]),
    (24, 3, [[0], [1, 2]] + [[3 * i, 3 * i + 1, 3 * i + 2] for i in range(1, 7)] + [[21, 22], [23]]),
    (2, 2, [[0], [1]]),
])
def test_small_plans(L, N, expect):
    assert default_group_plan(L, N) == expect


def test_bad_plans_rejected():
    with pytest.raises(ValueError):
        plan_offsets([[0], [2], [1]])
    with pytest.raises(ValueError):
        plan_offsets([[0], []])
