"""Sliding-window frame bookkeeping (integer, exact).

TEST INFRASTRUCTURE ONLY (see the package docstring).

VideoMLA paper, section 1 and appendix D.4: the cache is a fixed-size sliding
window of latent frames; the oldest frame leaves when a new one arrives, and
the long-horizon cache also pins sink frames.  Readings taken here: eviction is
per frame and first-in first-out; the first S frames (S = sink_frames, 0 by
default) stay in slots 0..S-1 for good; frame f >= S lives in slot
S + (f - S) mod W of the W-slot ring, so the frame written into a slot is
exactly the one that evicts the slot's previous occupant (f - W).
"""
from __future__ import annotations


class RingModel:
    def __init__(self, window_frames: int, tokens_per_frame: int, sink_frames: int = 0):
        if window_frames <= 0 or tokens_per_frame <= 0 or sink_frames < 0:
            raise ValueError("window and frame size must be positive")
        self.W = window_frames
        self.S = sink_frames
        self.T = tokens_per_frame
        self.n = 0  # frames appended so far

    def slot(self, frame: int) -> int:
        return frame if frame < self.S else self.S + (frame - self.S) % self.W

    def row(self, frame: int, token: int) -> int:
        return self.slot(frame) * self.T + token

    def valid_frames(self) -> list:
        """Frames held, in context order: sink frames, then the window (oldest first)."""
        sink = list(range(min(self.n, self.S)))
        return sink + list(range(max(self.S, self.n - self.W), self.n))

    def valid_rows(self) -> int:
        return len(self.valid_frames()) * self.T

    def append(self, chunk_frames: int) -> list:
        """Append frames [n, n+C); returns [(frame, slot)] in write order."""
        if chunk_frames > self.W:
            raise ValueError("a chunk may not exceed the window")
        written = [(f, self.slot(f)) for f in range(self.n, self.n + chunk_frames)]
        self.n += chunk_frames
        return written

    def slot_map(self) -> dict:
        """slot -> frame for every occupied slot."""
        return {self.slot(f): f for f in self.valid_frames()}
