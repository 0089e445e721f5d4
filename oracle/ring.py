"""Integer model of the encoder KV ring and the decoder modulo ring.

Encoder ring (streaming-plan page, "SHIPPED" section, "Unbounded length"
paragraph; family doc, Streaming row item 4): a 1536-slot ring written
contiguously; when it fills, the last 750 frames are copied to the front;
feeds are pushed in sub-batches of at most 512 frames so one feed can never
overflow it; ``abs_base`` is the absolute position held in slot 0, and the
mask works on absolute positions.

Readings where the pages leave a step open:
* split: a feed of n frames is cut greedily from its front into
  ceil(n/512) sub-batches, all of 512 frames but the last;
* trigger: compaction runs before a sub-batch of n frames exactly when
  n_kv + n > slots ("when the ring fills");
* kept rows: the last min(n_kv, window) frames (750, not 749: "copy the last
  750 frames"); the oldest kept row is masked for every later query, which
  is harmless.

Decoder ring (family doc, Streaming row item 5): token ``cur`` goes to slot
``cur % n_ctx``; positions stay absolute; with n_ctx = window = 8192 the slot
being overwritten holds cur - 8192, one past the window.  The same model
describes the encoder cache kept as a modulo ring instead of a compacting
one (every position p lives in slot p % slots).
"""
from __future__ import annotations

from dataclasses import dataclass, field


def split_feed(n: int, max_batch: int) -> list[int]:
    """Sub-batch sizes for a feed of n frames: greedy, <= max_batch each."""
    if n <= 0:
        return []
    full, rest = divmod(n, max_batch)
    return [max_batch] * full + ([rest] if rest else [])


@dataclass
class Compaction:
    n_kv_before: int      # rows held before the copy
    shift: int            # rows dropped from the front (= n_kv_before - kept)
    kept: int             # rows copied to slots [0, kept)
    abs_base_after: int


@dataclass
class EncRing:
    window: int = 750
    slots: int = 1536
    max_batch: int = 512
    abs_base: int = 0
    n_kv: int = 0
    events: list = field(default_factory=list)

    def reset(self, start_pos: int) -> None:
        self.abs_base, self.n_kv, self.events = int(start_pos), 0, []

    def needs_compaction(self, n: int) -> bool:
        return self.n_kv + n > self.slots

    def compact(self) -> Compaction | None:
        """Keep the last min(n_kv, window) rows at the front (a no-op when
        n_kv <= window)."""
        if self.n_kv <= self.window:
            return None
        kept = self.window
        shift = self.n_kv - kept
        self.abs_base += shift
        ev = Compaction(self.n_kv, shift, kept, self.abs_base)
        self.n_kv = kept
        self.events.append(ev)
        return ev

    def append(self, n: int) -> tuple[int, int]:
        """Append n frames (n <= max_batch); compact first if they would not
        fit.  Returns (first slot written, absolute position of that slot)."""
        if n > self.max_batch:
            raise ValueError("sub-batch larger than max_batch")
        if self.needs_compaction(n):
            self.compact()
        s0 = self.n_kv
        self.n_kv += n
        return s0, self.abs_base + s0

    def feed(self, n: int) -> list[tuple[int, int, int]]:
        """A whole feed: returns [(n_sub, first slot, first position)]."""
        return [(m,) + self.append(m) for m in split_feed(n, self.max_batch)]

    def slot_positions(self) -> list[int]:
        """Absolute position held by each occupied slot (slot s: abs_base+s)."""
        return [self.abs_base + s for s in range(self.n_kv)]

    @property
    def next_pos(self) -> int:
        return self.abs_base + self.n_kv


@dataclass
class DecRing:
    slots: int = 8192
    next_pos: int = 0

    def reset(self, start_pos: int = 0) -> None:
        self.next_pos = int(start_pos)

    def slot(self, pos: int) -> int:
        return pos % self.slots

    def append(self, n: int) -> list[tuple[int, int]]:
        """Positions written and their slots, in order."""
        out = [(p, p % self.slots) for p in range(self.next_pos, self.next_pos + n)]
        self.next_pos += n
        return out
