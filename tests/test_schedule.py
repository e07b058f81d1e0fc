"""The look-ahead schedule model (the review's Algorithm 1), CPU only."""
import itertools

import pytest

from oracle import schedule as sch


@pytest.mark.parametrize("s,e,w", list(itertools.product([0, 3, 16], [0, 1, 5, 16, 37], [1, 2, 4, 8])))
def test_every_block_once_and_lookahead_is_own_next(s, e, w):
    e = s + e
    groups = sch.group_schedule(s, e, w)
    seen = sorted(j for ev in groups.values() for _, j, _ in ev)
    assert seen == list(range(s, e))
    for wave, ev in groups.items():
        for k, (it, j, ahead) in enumerate(ev):
            assert it == k and (j - s) % w == wave
            if k + 1 < len(ev):
                assert ahead == ev[k + 1][1] == j + w
            else:
                assert ahead is None
            assert ahead is None or ahead < e


def test_four_warp_example():
    # warp 0 computes 0, 4, 8, ... and, while on 0, fetches 4; on 4 it fetches 8
    ev = sch.wave_schedule(0, 12, 4, 0)
    assert ev == [(0, 0, 4), (1, 4, 8), (2, 8, None)]
    tr = sch.expected_trace(0, 12, 4)
    assert tr[0] == [0, 0, -1] and tr[4] == [0, 1, 0] and tr[9] == [1, 2, 1]


@pytest.mark.parametrize("w,k", [(1, 2), (4, 2), (4, 3), (2, 8)])
def test_longer_lookahead_targets_the_same_wave_k_iterations_later(w, k):
    s, e = 5, 5 + 61
    for wave, ev in sch.group_schedule(s, e, w, k).items():
        for n, (it, j, ahead) in enumerate(ev):
            if n + k < len(ev):
                assert ahead == ev[n + k][1] == j + k * w
            else:
                assert ahead is None
    tr = sch.expected_trace(s, e, w, k)
    fetched = [j for j in range(s, e) if tr[j][2] >= 0]
    assert fetched == list(range(s + k * w, e))


def test_balanced_split_model():
    # uniform counts: the same partitions as a fixed split into slots/B parts
    size, parts = sch.balanced_split([64] * 8, 16, 64, 8, 32, 4)
    assert size == 16 and len(parts) == 32
    assert [p[2:] for p in parts[:4]] == [(0, 16), (16, 32), (32, 48), (48, 64)]
    # ragged: the smallest step multiple that fits; empty sequences get none
    size, parts = sch.balanced_split([100, 0, 7, 33], 16, 104, 8, 6, 6)
    assert size == 40  # 32 would need 4 + 1 + 2 = 7 > 6 partitions
    assert [(b, i) for b, i, _, _ in parts] == [(0, 0), (0, 1), (0, 2), (2, 0), (3, 0)]
    assert parts[2][2:] == (80, 100)
    for b, i, s, e in parts:
        assert s == i * size and s < e
    covered = {b: sum(e - s for bb, _, s, e in parts if bb == b) for b in range(4)}
    assert covered == {0: 100, 1: 0, 2: 7, 3: 33}

    # the per-sequence cap: slots would allow 16-block partitions, but the
    # workspace holds at most 4 per sequence
    size, parts = sch.balanced_split([100, 0, 0, 0], 16, 104, 8, 64, 4)
    assert size == 32 and len(parts) == 4


def test_balanced_split_keeps_the_reduce_rule():
    # 12 partitions of 16 would fit the slots, but more than 8 partitions
    # need at least 64 blocks each: 3 of 64 instead (sizes step by 8)
    size, parts = sch.balanced_split([190], 16, 192, 8, 100, 100)
    assert size == 24  # 24 gives ceil(190 / 24) = 8 partitions
    size, parts = sch.balanced_split([1000], 16, 1024, 8, 100, 100)
    assert size == 64 and len(parts) == 16
