"""Model of the look-ahead block schedule, for checking the kernel's trace.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The asynchronous-KV-prefetch review (section 3.4, Algorithm 1) gives each of
w warps of a thread block a block-index range [s, e): a warp walks its blocks
with stride w, looks up the current block in the block table and loads it,
and, when the block w further on still lies inside the range, looks that one
up too and starts fetching it into the cache before computing Q*K^T on the
current one.  The
third page (section 2.2) assigns warp i the blocks i, i + 4, i + 8, ... of a
4-warp block, so wave i starts at s + i.
"""
from typing import Dict, List, Optional, Sequence, Tuple

Event = Tuple[int, int, Optional[int]]  # (iteration, computed block, fetched-ahead block)


def wave_schedule(s: int, e: int, w: int, wave: int, distance: int = 1) -> List[Event]:
    """Events of one wave, in program order.  The wave's blocks are the
    arithmetic progression s + wave, s + wave + w, ... below e; in its n-th
    iteration it computes the n-th of them and fetches ahead the block
    distance * w further on, if that one is still below e (the review's
    Algorithm 1 is distance 1)."""
    if w <= 0 or not 0 <= wave < w or distance < 1:
        raise ValueError("need 0 <= wave < w and distance >= 1")
    blocks = range(s + wave, e, w)
    return [(n, j, j + distance * w if j + distance * w < e else None)
            for n, j in enumerate(blocks)]


def group_schedule(s: int, e: int, w: int, distance: int = 1) -> Dict[int, List[Event]]:
    """Events of all w waves of one work-group over [s, e)."""
    return {wave: wave_schedule(s, e, w, wave, distance) for wave in range(w)}


def expected_trace(s: int, e: int, w: int, distance: int = 1):
    """Per block j in [s, e): (wave that computes it, its iteration, wave that
    fetched it ahead or -1).  This is what the kernel's debug trace records."""
    out = {}
    for wave, events in group_schedule(s, e, w, distance).items():
        for it, j, _ in events:
            out[j] = [wave, it, -1]
    for wave, events in group_schedule(s, e, w, distance).items():
        for _, _, ahead in events:
            if ahead is not None:
                out[ahead][2] = wave
    return out


def balanced_split(block_counts: Sequence[int], pb_min: int, pb_max: int, step: int,
                   slots: int, max_parts: int, few: int = 8,
                   big: int = 64) -> Tuple[int, List[Tuple[int, int, int, int]]]:
    """The launch's balanced split of ragged sequences (not a step of the
    method: which work-group walks which block range).  The partition size is
    the smallest multiple of `step` in [pb_min, pb_max] with which all
    sequences together need at most `slots` partitions, none needs more than
    `max_parts`, and none more than `few` unless the size is at least `big`;
    the partitions are listed sequence by sequence.  Returns (size,
    [(sequence, index, s, e)]) with each range [s, e) of block indices;
    sequences without blocks get none.  Written from that definition by plain
    enumeration."""
    size = None
    for pb in range(pb_min, pb_max + 1, step):
        most = max([-(-n // pb) for n in block_counts] + [0])
        if (sum(-(-n // pb) for n in block_counts) <= slots and most <= max_parts and
                (most <= few or pb >= big)):
            size = pb
            break
    if size is None:
        raise ValueError("no partition size fits the slots")
    parts = []
    for b, n in enumerate(block_counts):
        for i, s in enumerate(range(0, n, size)):
            parts.append((b, i, s, min(n, s + size)))
    assert len(parts) <= slots
    return size, parts
