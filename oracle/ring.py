"""Bounded per-rollout KV cache bookkeeping, kept as a deque (test infrastructure only).

Pages:
* FlashDreams blog post, "Bounded Memory for Infinite Rollouts": one cache
  per rollout, bounded VRAM for arbitrarily long rollouts, eviction handled
  inside the framework.
* Cosmos3-H-Dreams model card, "Model Architecture": the conditioning frame is
  prefilled into the KV cache once; "Software Integration": static-shape KV
  cache.
* AlpaDreams write-up, section VI: the model keeps the first frame plus a
  cache of subsequent historical frames.

Reading taken where the pages are silent: the cache holds S persistent
"sink" frames (the first S committed frames of a sequence, never evicted)
plus a FIFO window of the W most recent later frames.  Storage is S + W
fixed slots.  A new window frame takes the slot freed by the frame it evicts
(the oldest window frame) or, while the window is filling, the lowest free
window slot.  With W == 0 later frames are not stored at all.

This module derives slots by simulation; the closed forms used by the
library are checked against it in the tests.
"""

from collections import deque


class DequeRing:
    """One rollout's cache state: sink list + window deque + free-slot set."""

    def __init__(self, n_sink, window):
        if n_sink < 0 or window < 0:
            raise ValueError("n_sink and window must be >= 0")
        self.n_sink = n_sink
        self.window = window
        self.reset()

    def reset(self):
        self.sinks = []                 # [(frame, slot)] in commit order
        self.win = deque()              # [(frame, slot)] oldest first
        self.free = set(range(self.n_sink, self.n_sink + self.window))
        self.n_committed = 0

    def commit(self):
        """Commit the next frame id; return (frame, slot, evicted_frames).

        slot is -1 when the frame is not stored (W == 0, non-sink frame).
        """
        frame = self.n_committed
        self.n_committed += 1
        evicted = []
        if len(self.sinks) < self.n_sink:
            slot = len(self.sinks)
            self.sinks.append((frame, slot))
            return frame, slot, evicted
        if self.window == 0:
            return frame, -1, evicted
        if len(self.win) == self.window:
            old_frame, slot = self.win.popleft()
            evicted.append(old_frame)
        else:
            slot = min(self.free)
            self.free.remove(slot)
        self.win.append((frame, slot))
        return frame, slot, evicted

    def retained(self):
        """[(frame, slot)] of every stored frame, in temporal order."""
        return list(self.sinks) + list(self.win)

    def retained_frames(self):
        return [f for f, _ in self.retained()]
