"""Pins for the oracle's deque ring (CPU).

The deque simulation in ``oracle.ring`` is checked against closed forms
written out here, against a hand-derived worked example, and against the
invariants of a bounded FIFO cache (FlashDreams blog post, "Bounded Memory
for Infinite Rollouts": a per-rollout cache whose size does not grow).
"""

import os

import pytest

from oracle.ring import DequeRing
from oracle.attention import visible_frames

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def closed_slot(f, S, W):
    if f < S:
        return f
    if W == 0:
        return -1
    return S + (f - S) % W


def closed_retained(m, S, W):
    """Frames stored after committing ids 0..m."""
    sinks = list(range(min(S, m + 1)))
    win = list(range(max(S, m + 1 - W), m + 1)) if W > 0 else []
    return sinks + win


def closed_evicted(m, S, W):
    """Frames evicted by committing frame m."""
    if W > 0 and m >= S + W:
        return [m - W]
    return []


@pytest.mark.parametrize("S", range(0, 7))
@pytest.mark.parametrize("W", range(0, 7))
def test_deque_matches_closed_form(S, W):
    r = DequeRing(S, W)
    seen_evicted = []
    for m in range(3 * (S + W) + 20):
        frame, slot, ev = r.commit()
        assert frame == m
        assert slot == closed_slot(m, S, W)
        assert ev == closed_evicted(m, S, W)
        assert r.retained_frames() == closed_retained(m, S, W)
        for f, s in r.retained():
            assert s == closed_slot(f, S, W)
        slots = [s for _, s in r.retained()]
        assert len(set(slots)) == len(slots)          # no two frames share a slot
        assert all(0 <= s < S + W for s in slots)
        seen_evicted.extend(ev)
    assert seen_evicted == sorted(seen_evicted)       # FIFO: strictly increasing
    assert all(e >= S for e in seen_evicted)          # sinks never evicted


@pytest.mark.parametrize("S,W", [(1, 3), (1, 18), (1, 17), (2, 5), (0, 4), (3, 0)])
def test_bounded_after_10000_steps(S, W):
    r = DequeRing(S, W)
    for m in range(10_000):
        r.commit()
        assert len(r.retained()) <= S + W
    assert len(r.retained()) == S + W if W > 0 else min(S, 10_000)
    assert r.retained_frames() == closed_retained(9_999, S, W)


def test_worked_example():
    rows = []
    with open(os.path.join(GOLDEN, "ring_tiny_worked_example.txt")) as fh:
        for line in fh:
            if line.startswith("#") or not line.strip():
                continue
            rows.append([c.strip() for c in line.split("|")])
    S, W, ft = 1, 3, 16
    r = DequeRing(S, W)
    for frame_s, vis_s, nk_s, slot_s, ev_s, ret_s in rows:
        n0 = int(frame_s)
        vis = visible_frames(n0, 1, S, W)
        assert vis == [int(v) for v in vis_s.split(",")]
        assert len(vis) * ft == int(nk_s)
        frame, slot, ev = r.commit()
        assert frame == n0 and slot == int(slot_s)
        assert ev == ([] if ev_s == "-" else [int(ev_s)])
        assert r.retained_frames() == [int(v) for v in ret_s.split(",")]


def test_reset_starts_new_sequence():
    r = DequeRing(1, 2)
    for _ in range(7):
        r.commit()
    r.reset()
    assert r.retained() == [] and r.n_committed == 0
    assert r.commit() == (0, 0, [])


@pytest.mark.parametrize("S,W,C", [(1, 3, 1), (1, 18, 3), (2, 2, 4), (0, 3, 4), (1, 1, 3)])
def test_visible_frames_match_retained(S, W, C):
    """Keys of a chunk = frames retained before it + the chunk itself."""
    r = DequeRing(S, W)
    n0 = 0
    for _ in range(12):
        vis = visible_frames(n0, C, S, W)
        assert vis == r.retained_frames() + list(range(n0, n0 + C))
        for _ in range(C):
            r.commit()
        n0 += C
