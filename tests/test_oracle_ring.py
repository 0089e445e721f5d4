"""Pins for the integer ring model (oracle/ring.py): closed-form compaction
schedules, the slot/position invariant, the pages' own compaction counts
(tests/golden/ring_page_figures.json) and the decoder modulo ring."""
import json
import os

import pytest

from oracle.ring import EncRing, DecRing, split_feed

GOLD = os.path.join(os.path.dirname(__file__), "golden", "ring_page_figures.json")


def test_split_feed():
    assert split_feed(0, 512) == []
    assert split_feed(4, 512) == [4]
    assert split_feed(512, 512) == [512]
    assert split_feed(750, 512) == [512, 238]
    assert split_feed(15300, 512) == [512] * 29 + [452]


def test_catch_up_schedule_closed_form():
    # 15300 frames in 512-frame batches: ring holds 512, 1024, 1536 after the
    # first three; every later batch needs a compaction (27 in total).
    r = EncRing()
    seen = []
    for i, m in enumerate(split_feed(15300, 512)):
        before = len(r.events)
        r.append(m)
        if len(r.events) > before:
            seen.append(i)
    assert seen == list(range(3, 30))
    assert len(r.events) == 27
    assert r.events[0].n_kv_before == 1536 and r.events[0].shift == 786
    assert all(e.n_kv_before == 1262 and e.shift == 512 for e in r.events[1:])
    # every later copy overlaps its source (shift < kept)
    assert sum(e.shift < e.kept for e in r.events) == 26
    assert r.n_kv == 750 + 452 and r.next_pos == 15300


def test_steady_state_schedule_closed_form():
    # pre-filled to 750 then 4 frames per step: compaction when 750+4k+4 > 1536,
    # i.e. at steps 196, 392, ... (period 196)
    r = EncRing()
    r.reset(123_456)
    r.feed(750)
    assert r.n_kv == 750 and not r.events
    steps = []
    for s in range(1000):
        before = len(r.events)
        r.feed(4)
        if len(r.events) > before:
            steps.append(s)
    assert steps == [196, 392, 588, 784, 980]
    assert all(e.shift == 784 for e in r.events)


def test_slot_position_invariant():
    r = EncRing()
    r.reset(50)
    fed = 0
    for m in [3, 7, 500, 512, 1, 4, 300, 512, 512, 2]:
        r.feed(m)
        fed += m
        assert r.slot_positions() == list(range(r.abs_base, r.abs_base + r.n_kv))
        assert r.n_kv <= r.slots
        assert r.slot_positions()[-1] == 50 + fed - 1


def test_explicit_compact():
    r = EncRing()
    r.feed(800)
    assert r.compact().shift == 50
    assert r.abs_base == 50 and r.n_kv == 750
    assert r.compact() is None   # n_kv <= window: no-op


def test_positions_follow_feeds():
    r = EncRing()
    r.reset(7)
    total = 0
    for m in [1, 2, 3, 511, 512, 513, 4, 4, 1000]:
        r.feed(m)
        total += m
        assert r.next_pos == 7 + total
        assert r.abs_base + r.n_kv == 7 + total
        assert r.n_kv >= min(total, 750)


@pytest.mark.parametrize("clip", json.load(open(GOLD))["clips"], ids=lambda c: c["name"])
def test_page_compaction_counts(clip):
    for f in clip["feed_frames"]:
        r = EncRing()
        left = clip["frames"]
        while left > 0:
            m = min(f, left)
            r.feed(m)
            left -= m
        assert clip["min_compactions"] <= len(r.events) <= clip["max_compactions"], (f, len(r.events))


def test_decoder_modulo_ring():
    d = DecRing(8192)
    w = d.append(39)
    assert w[0] == (0, 0) and w[-1] == (38, 38)
    d.reset(8190)
    w = d.append(4)
    assert [s for _, s in w] == [8190, 8191, 0, 1]
    # the slot written by cur holds cur - 8192 before: one past the window
    assert d.slot(10_000) == d.slot(10_000 - 8192)
