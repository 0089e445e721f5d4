"""CPU tests of the host logic behind every entry point, with the library's
testing hook in dry-run mode: no kernel is launched (device pointers are fake
and never touched), launches are counted, and one chosen launch can be made
to fail as a failed launch would.

What is checked (streaming-plan page, "Per-hook behavior": validation is pure
and precedes any mutation; reset clears streaming state and keeps the
allocations):
* argument errors enqueue nothing and change no state;
* a failed launch at any point of a call returns VRT_ERR_DEVICE and poisons
  every state of the call; poisoned states refuse later calls before
  enqueueing anything; reset clears the poison;
* the attention half of a block poisons its states when its output
  projection fails after the path has appended the feed's rows, and refuses
  lookahead states up front;
* a conv stem is left as it was when any launch of its feed fails;
* the host mirror that dry runs advance follows the oracle's ring model, and
  each feed makes the launches its plan says (fused append on the vector
  path, separate append on the matrix path, one compaction launch)."""
import pytest

import sliding_window_cached_amd as vrt
from oracle.ring import EncRing

FAKE = 1 << 40          # 256-byte aligned, never dereferenced in dry-run mode
Q, K, V, O, WS = (FAKE + (i + 1) * (1 << 36) for i in range(5))


@pytest.fixture(autouse=True)
def dry_hook():
    vrt.test_launch_hook(0, dry_run=True)
    yield
    vrt.test_launch_hook(0, dry_run=False)


def states_of(desc, n, starts=None):
    nb = vrt.state_device_bytes(desc)
    return [vrt.StreamState(desc, FAKE + i * ((nb + 255) // 256 * 256), nb,
                            0 if starts is None else starts[i]) for i in range(n)]


def poisoned(st) -> bool:
    return st.status() == vrt.ERR_POISONED


def test_dry_run_counts_launches_and_follows_the_ring_model():
    d = vrt.enc_desc(dtype=vrt.BF16, n_layers=2)
    sts = states_of(d, 3, [0, 10, 999_000])
    r = EncRing()
    r.reset(0)
    # 4-frame feeds: one fused launch each, plus one compaction launch when due
    for i in range(400):
        before = len(r.events)
        r.feed(4)
        vrt.test_launch_hook(0, dry_run=True)
        vrt.enc_attn_feed(sts, 0, 2, Q, K, V, 4, O)
        assert vrt.test_launch_count() == 1 + (len(r.events) - before), i
    for j, s in enumerate(sts):
        base, nkv = s.query(1)
        assert nkv == r.n_kv and base - [0, 10, 999_000][j] == r.abs_base
    # a 1300-frame feed: sub-batches 512, 512, 276 on the matrix path, each a
    # separate append and an attention launch, compactions where the model has them
    before = len(r.events)
    r.feed(1300)
    vrt.test_launch_hook(0, dry_run=True)
    vrt.enc_attn_feed(sts, 0, 2, Q, K, V, 1300, O)
    assert vrt.test_launch_count() == 3 * 2 + (len(r.events) - before)
    assert sts[0].query(0) == (r.abs_base, r.n_kv)


def test_argument_errors_enqueue_nothing():
    d = vrt.enc_desc(dtype=vrt.BF16, n_layers=2)
    sts = states_of(d, 2)
    other = states_of(vrt.enc_desc(dtype=vrt.F32, n_layers=2), 1)[0]
    dec = states_of(vrt.dec_desc(), 1)[0]
    bad = [
        lambda: vrt.enc_attn_feed(sts, 0, 2, 0, K, V, 4, O, check=False),        # null q
        lambda: vrt.enc_attn_feed(sts, 0, 2, Q, K, V, 0, O, check=False),        # no frames
        lambda: vrt.enc_attn_feed(sts, 1, 2, Q, K, V, 4, O, check=False),        # layer range
        lambda: vrt.enc_attn_feed(sts + [other], 0, 1, Q, K, V, 4, O, check=False),  # mixed descs
        lambda: vrt.enc_attn_feed([sts[0], sts[0]], 0, 1, Q, K, V, 4, O, check=False),  # repeated
        lambda: vrt.enc_attn_feed([dec], 0, 1, Q, K, V, 4, O, check=False),      # decoder state
        lambda: vrt.dec_attn_step([dec], 0, 1, Q, K, V, 1, O, WS, 16, check=False),   # short ws
        lambda: vrt.dec_attn_step(sts, 0, 1, Q, K, V, 1, O, WS, 1 << 30, check=False),  # encoder
    ]
    for i, call in enumerate(bad):
        vrt.test_launch_hook(0, dry_run=True)
        assert call() != vrt.OK, i
        assert vrt.test_launch_count() == 0, i
    assert sts[0].query(0) == (0, 0) and dec.query(0) == (0, 0)
    assert not poisoned(sts[0]) and not poisoned(dec)


@pytest.mark.parametrize("n_new", [4, 1300])
def test_launch_failure_poisons_every_state_and_reset_clears(n_new):
    d = vrt.enc_desc(dtype=vrt.BF16, n_layers=2)
    # how many launches the call makes when nothing fails
    probe = states_of(d, 3)
    for s in probe:
        vrt.enc_attn_feed([s], 0, 2, Q, K, V, 1536, O)     # fill the rings: the next feed compacts
    vrt.test_launch_hook(0, dry_run=True)
    vrt.enc_attn_feed(probe, 0, 2, Q, K, V, n_new, O)
    n_launch = vrt.test_launch_count()
    assert n_launch >= 2
    for k in range(1, n_launch + 1):
        sts = states_of(d, 3)
        for s in sts:
            vrt.enc_attn_feed([s], 0, 2, Q, K, V, 1536, O)
        vrt.test_launch_hook(k, dry_run=True)
        assert vrt.enc_attn_feed(sts, 0, 2, Q, K, V, n_new, O, check=False) == vrt.ERR_DEVICE, k
        assert vrt.test_launch_count() == k
        assert all(poisoned(s) for s in sts), k
        assert vrt.last_device_error() != ""
        # refused before anything is enqueued
        vrt.test_launch_hook(0, dry_run=True)
        assert vrt.enc_attn_feed(sts, 0, 2, Q, K, V, 4, O, check=False) == vrt.ERR_POISONED
        assert vrt.ring_compact_status(sts, 0, 2) == vrt.ERR_POISONED
        assert vrt.test_launch_count() == 0
        for s in sts:
            s.reset(5)
            assert not poisoned(s) and s.query(1) == (5, 0)
        assert vrt.enc_attn_feed(sts, 0, 2, Q, K, V, 4, O, check=False) == vrt.OK
        assert sts[2].query(0) == (5, 4)


def test_decoder_launch_failure_poisons():
    d = vrt.dec_desc(n_layers=2)
    sts = states_of(d, 2)
    wsb = vrt.dec_workspace_bytes(d, 2, 2, 1)
    vrt.dec_attn_step(sts, 0, 2, Q, K, V, 39, O)
    vrt.test_launch_hook(0, dry_run=True)
    vrt.dec_attn_step(sts, 0, 2, Q, K, V, 1, O, WS, wsb)
    assert vrt.test_launch_count() == 2          # split-K attention, then the merge
    for k in (1, 2):
        sts = states_of(d, 2)
        vrt.dec_attn_step(sts, 0, 2, Q, K, V, 39, O)
        vrt.test_launch_hook(k, dry_run=True)
        assert vrt.dec_attn_step(sts, 0, 2, Q, K, V, 1, O, WS, wsb, check=False) == vrt.ERR_DEVICE
        assert all(poisoned(s) for s in sts)
        assert vrt.dec_attn_step(sts, 0, 2, Q, K, V, 1, O, WS, wsb, check=False) == vrt.ERR_POISONED
        for s in sts:
            s.reset(0)
        assert vrt.dec_attn_step(sts, 0, 2, Q, K, V, 1, O, WS, wsb, check=False) == vrt.OK


def _block_args(desc, n_states, n_new):
    w = vrt.block_weights(FAKE + (7 << 36), FAKE + (8 << 36), None, None, FAKE + (9 << 36), None)
    wsb = vrt.block_workspace_bytes(desc, n_states * n_new)
    return w, wsb


def test_block_feed_poisons_on_any_failed_launch():
    d = vrt.enc_desc(dtype=vrt.BF16, n_layers=1)
    w, wsb = _block_args(d, 2, 4)
    sts = states_of(d, 2)
    vrt.test_launch_hook(0, dry_run=True)
    vrt.enc_block_feed(sts, 0, Q, 4, w, O, WS, wsb)
    n_launch = vrt.test_launch_count()
    assert n_launch == 4                  # norm, q/k/v product, fused attention, output product
    for k in range(1, n_launch + 1):
        sts = states_of(d, 2)
        vrt.test_launch_hook(k, dry_run=True)
        assert vrt.enc_block_feed(sts, 0, Q, 4, w, O, WS, wsb, check=False) == vrt.ERR_DEVICE, k
        assert all(poisoned(s) for s in sts), k
        if k == n_launch:   # the path ran: the rings already hold the feed's rows
            assert sts[0].query(0) == (0, 4)
        vrt.test_launch_hook(0, dry_run=True)
        assert vrt.enc_block_feed(sts, 0, Q, 4, w, O, WS, wsb, check=False) == vrt.ERR_POISONED
        assert vrt.test_launch_count() == 0


def test_block_feed_refuses_lookahead_states():
    d = vrt.lookahead_desc(16, 4)
    w, wsb = _block_args(d, 1, 4)
    sts = states_of(d, 1)
    vrt.test_launch_hook(0, dry_run=True)
    assert vrt.enc_block_feed(sts, 0, Q, 4, w, O, WS, wsb, check=False) == vrt.ERR_UNSUPPORTED
    assert vrt.test_launch_count() == 0
    assert sts[0].query(0) == (0, 0)


def test_conv_stem_is_unchanged_when_a_launch_fails():
    n_mel, dm = 128, 1280
    nb = vrt.conv_stem_device_bytes(n_mel, dm)
    w = vrt.conv_weights(FAKE + (7 << 36), None, FAKE + (8 << 36), None)
    for n_frames in (8, 1):     # with conv1 outputs, and without (pending 1 + 1 < 3)
        wsb = vrt.conv_workspace_bytes(n_mel, dm, 2, n_frames)
        stems = [vrt.ConvStem(n_mel, dm, FAKE + i * 4096, nb) for i in range(2)]
        vrt.test_launch_hook(0, dry_run=True)
        vrt.conv_stem_feed(stems, Q, n_frames, w, O, WS, wsb)
        n_launch = vrt.test_launch_count()
        after = stems[0].query()
        assert after[0] == n_frames
        for k in range(1, n_launch + 1):
            fresh = [vrt.ConvStem(n_mel, dm, FAKE + i * 4096, nb) for i in range(2)]
            vrt.test_launch_hook(k, dry_run=True)
            s = vrt.conv_stem_feed(fresh, Q, n_frames, w, O, WS, wsb, check=False)
            assert s == vrt.ERR_DEVICE, (n_frames, k)
            assert all(c.query() == (0, 1) for c in fresh), (n_frames, k)
            vrt.test_launch_hook(0, dry_run=True)
            assert vrt.conv_stem_feed(fresh, Q, n_frames, w, O, WS, wsb) >= 0
            assert fresh[1].query() == after


def test_static_decode_step_host_logic():
    """The allocation-free decode step: the same launches as the workspace
    step, and refused (nothing enqueued) past its 128 MiB of partials."""
    d = vrt.dec_desc(n_layers=26)
    sts = states_of(d, 2)
    vrt.dec_attn_step(sts, 0, 26, Q, K, V, 39, O)
    vrt.test_launch_hook(0, dry_run=True)
    assert vrt.dec_attn_step_static(sts, 0, 26, Q, K, V, 1, O, check=False) == vrt.OK
    assert vrt.test_launch_count() == 2 and sts[1].query(25) == (0, 40)
    per_state = vrt.dec_workspace_bytes(d, 1, 26, 1)
    big = states_of(d, (128 << 20) // per_state + 1)
    vrt.test_launch_hook(0, dry_run=True)
    assert vrt.dec_attn_step_static(big, 0, 26, Q, K, V, 1, O, check=False) == vrt.ERR_CAPACITY
    assert vrt.test_launch_count() == 0 and big[0].query(0) == (0, 0)
    assert vrt.dec_attn_step_static(big[:32], 0, 26, Q, K, V, 1, O, check=False) == vrt.OK


def test_decoder_workspace_must_be_16_byte_aligned():
    """A decode step with a misaligned or missing workspace is refused before
    anything is enqueued or any state moves; an aligned one goes through."""
    d = vrt.dec_desc(n_layers=1)
    sts = states_of(d, 2)
    vrt.dec_attn_step(sts, 0, 1, Q, K, V, 39, O)
    wsb = vrt.dec_workspace_bytes(d, 2, 1, 1)
    for bad in (WS + 4, WS + 8, None):
        vrt.test_launch_hook(0, dry_run=True)
        assert vrt.dec_attn_step(sts, 0, 1, Q, K, V, 1, O, bad, wsb, check=False) == vrt.ERR_INVALID
        assert vrt.test_launch_count() == 0
        assert all(s.query(0) == (0, 39) for s in sts)
    vrt.test_launch_hook(0, dry_run=True)
    assert vrt.dec_attn_step(sts, 0, 1, Q, K, V, 1, O, WS + 16, wsb, check=False) == vrt.OK
    assert vrt.test_launch_count() == 2 and all(s.query(0) == (0, 40) for s in sts)
