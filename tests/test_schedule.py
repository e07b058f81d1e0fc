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
