"""CPU tests of the C ABI: the library loads and exports every symbol the
public header declares, descriptors are checked as documented, the host ring
planner agrees with the oracle's ring model, and argument errors are caught
before anything is enqueued.  No compute call is made here (no GPU)."""
import ctypes
import os
import random
import re

import pytest

import sliding_window_cached_amd as vrt
from oracle.ring import DecRing, EncRing

HDR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "vrt.h")


def test_exports_every_declared_symbol():
    text = open(HDR).read()
    declared = set(re.findall(r"\b(vrt_[a-z_0-9]+)\s*\(", text))
    assert len(declared) >= 17
    lib = ctypes.CDLL(vrt.LIB_PATH)
    for name in sorted(declared):
        assert hasattr(lib, name), name
    assert declared == set(vrt.EXPORTS)


def test_version_and_status_strings():
    assert "gfx950" in vrt.version()
    for s in range(6):
        assert vrt.status_str(s)


def test_desc_checks():
    assert vrt.desc_check(vrt.enc_desc()) == vrt.OK
    assert vrt.desc_check(vrt.dec_desc()) == vrt.OK
    assert vrt.desc_check(vrt.enc_desc(head_dim=96)) == vrt.ERR_UNSUPPORTED
    assert vrt.desc_check(vrt.enc_desc(ring_slots=1261)) == vrt.ERR_UNSUPPORTED  # < W + max_batch
    assert vrt.desc_check(vrt.enc_desc(ring_slots=1262)) == vrt.OK
    assert vrt.desc_check(vrt.dec_desc(ring_slots=8000)) == vrt.ERR_UNSUPPORTED  # < window
    assert vrt.desc_check(vrt.dec_desc(ring_slots=8200)) == vrt.ERR_UNSUPPORTED  # not 64-multiple
    assert vrt.desc_check(vrt.dec_desc(ring_slots=16384)) == vrt.OK
    d = vrt.enc_desc()
    d.lookahead = 1                      # only for ENC_LOOKAHEAD
    assert vrt.desc_check(d) == vrt.ERR_INVALID
    assert vrt.desc_check(vrt.enc_desc(heads=0)) == vrt.ERR_INVALID
    assert vrt.desc_check(vrt.dec_desc(heads_q=30)) == vrt.ERR_INVALID  # not a multiple of 8
    assert vrt.desc_check(vrt.dec_desc(heads_q=256, heads_kv=8)) == vrt.ERR_UNSUPPORTED  # group 32
    bad = vrt.enc_desc()
    bad.dtype = 7
    assert vrt.desc_check(bad) == vrt.ERR_UNSUPPORTED
    # heads narrower than 64 only without rotation (the moonshine encoder's 8 x 40)
    assert vrt.desc_check(vrt.lookahead_desc(16, 4, head_dim=40)) == vrt.OK
    assert vrt.desc_check(vrt.lookahead_desc(16, 4, head_dim=8)) == vrt.OK
    assert vrt.desc_check(vrt.lookahead_desc(16, 4, head_dim=36)) == vrt.ERR_UNSUPPORTED
    assert vrt.desc_check(vrt.lookahead_desc(16, 4, head_dim=96)) == vrt.ERR_UNSUPPORTED
    assert vrt.desc_check(vrt.enc_desc(head_dim=40)) == vrt.ERR_UNSUPPORTED
    assert vrt.desc_check(vrt.dec_desc(head_dim=40)) == vrt.ERR_UNSUPPORTED


def test_state_bytes_and_offsets():
    d = vrt.enc_desc(n_layers=32)
    assert vrt.state_device_bytes(d) == 32 * 2 * 20 * 1536 * 64 * 2
    dd = vrt.dec_desc(n_layers=26)
    assert vrt.state_device_bytes(dd) == 26 * 2 * 8 * 8192 * 128 * 2
    sl = 1536 * 64 * 2
    assert vrt.ring_offset(d, 0, 0, 0) == 0
    assert vrt.ring_offset(d, 0, 1, 0) == 20 * sl
    assert vrt.ring_offset(d, 3, 1, 5) == 3 * 40 * sl + 25 * sl
    assert vrt.ring_offset(d, 32, 0, 0) == 2 ** 64 - 1
    assert vrt.offline_scratch_bytes(d, 1000) == 2 * 20 * 1000 * 64 * 2
    # a 40-wide lookahead head: ring rows padded to 64, waiting q rows 40 wide
    la = vrt.lookahead_desc(16, 4, n_layers=6, head_dim=40)
    assert vrt.state_device_bytes(la) == 6 * (2 * 8 * la.ring_slots * 64 * 2 + 3 * 8 * 40 * 2)
    assert vrt.ring_offset(la, 1, 1, 2) == (2 * 8 * la.ring_slots * 64 * 2) + 10 * la.ring_slots * 64 * 2
    assert vrt.offline_scratch_bytes(la, 100) == 2 * 8 * 100 * 64 * 2


def test_ring_advance_matches_oracle_model():
    d = vrt.enc_desc()
    rng = random.Random(0)
    for trial in range(200):
        r = EncRing()
        start = rng.randrange(0, 10 ** 6)
        r.reset(start)
        base, nkv = start, 0
        for _ in range(rng.randrange(1, 40)):
            n = rng.choice([1, 2, 3, 4, 7, 31, 32, 100, 511, 512, 513, 750, 1536, 2000])
            before = len(r.events)
            r.feed(n)
            base, nkv, nc = vrt.ring_advance(d, base, nkv, n)
            assert (base, nkv) == (r.abs_base, r.n_kv)
            assert nc == len(r.events) - before


def test_attn_path_is_a_function_of_desc_and_n():
    f32, bf = vrt.enc_desc(dtype=vrt.F32), vrt.enc_desc(dtype=vrt.BF16)
    for n in (1, 4, 16, 31, 32, 512, 15300):
        assert vrt.attn_path(f32, n) == 0
        assert vrt.attn_path(bf, n) == (1 if n >= 32 else 0)
        assert vrt.attn_path(vrt.dec_desc(), n) == 0                  # GQA decoder
        assert vrt.attn_path(vrt.enc_desc(head_dim=128), n) == 0
    assert vrt.attn_path(bf, 0) == -1
    bad = vrt.enc_desc()
    bad.lookahead = 3
    assert vrt.attn_path(bad, 64) == -1


# A 256-byte aligned fake address: valid for host bookkeeping, never touched,
# because every call below fails its argument checks before enqueueing.
FAKE = 1 << 40


def _state(desc, start=0):
    return vrt.StreamState(desc, FAKE, vrt.state_device_bytes(desc), start)


def test_create_reset_query_host_only():
    d = vrt.enc_desc(n_layers=3)
    st = _state(d, 42)
    assert st.query(0) == (42, 0) and st.query(2) == (42, 0)
    st.reset(7)
    assert st.query(1) == (7, 0)
    with pytest.raises(vrt.VrtError) as e:
        st.query(3)
    assert e.value.status == vrt.ERR_INVALID
    with pytest.raises(vrt.VrtError) as e:
        vrt.StreamState(d, FAKE, vrt.state_device_bytes(d) - 1, 0)
    assert e.value.status == vrt.ERR_CAPACITY
    with pytest.raises(vrt.VrtError) as e:
        vrt.StreamState(d, FAKE + 8, vrt.state_device_bytes(d), 0)   # misaligned
    assert e.value.status == vrt.ERR_INVALID
    with pytest.raises(vrt.VrtError) as e:
        vrt.StreamState(d, FAKE, vrt.state_device_bytes(d), -1)
    assert e.value.status == vrt.ERR_INVALID


def test_feed_argument_errors_enqueue_nothing():
    d = vrt.enc_desc(n_layers=2)
    a, b = _state(d), _state(d)
    other = _state(vrt.enc_desc(n_layers=3))
    dec = _state(vrt.dec_desc(n_layers=2))
    P = FAKE
    cases = [
        ([a], 0, 1, None, 4),        # null q
        ([a], 0, 1, P, 0),           # n_new = 0
        ([a], 1, 2, P, 4),           # layer range past n_layers
        ([a], -1, 1, P, 4),
        ([a, a], 0, 1, P, 4),        # repeated state
        ([a, other], 0, 1, P, 4),    # mixed descs
        ([dec], 0, 1, P, 4),         # decoder state into the encoder feed
    ]
    for states, l0, nl, q, n in cases:
        s = vrt.enc_attn_feed(states, l0, nl, q, P, P, n, P, 0, check=False)
        assert s == vrt.ERR_INVALID, (l0, nl, q, n)
    for st in (a, b):
        assert st.query(0) == (0, 0) and st.query(1) == (0, 0)
    with pytest.raises(vrt.VrtError):
        vrt.ring_compact([dec], 0, 1)


def test_decoder_argument_errors():
    d = vrt.dec_desc(n_layers=1, window=256, ring_slots=256)
    st = _state(d)
    P = FAKE
    ws = vrt.dec_workspace_bytes(d, 1, 1, 1)
    assert ws > 0
    # missing workspace for a decode step
    assert vrt.dec_attn_step([st], 0, 1, P, P, P, 1, P, None, 0, check=False) == vrt.ERR_INVALID
    assert vrt.dec_attn_step([st], 0, 1, P, P, P, 1, P, P, ws - 4, check=False) == vrt.ERR_CAPACITY
    # a 300-token prefill on a 256-slot ring would overwrite keys its own
    # first queries need
    assert vrt.dec_attn_step([st], 0, 1, P, P, P, 300, P, check=False) == vrt.ERR_INVALID
    assert st.query(0) == (0, 0)


def test_position_limit():
    """Absolute positions stay below 2^31: creation at 2^31 and feeds whose
    frames would reach it are refused before anything is enqueued."""
    d = vrt.enc_desc()
    lim = 2 ** 31
    with pytest.raises(vrt.VrtError) as e:
        _state(d, lim)
    assert e.value.status == vrt.ERR_INVALID
    st = _state(d, lim - 3)
    P = FAKE
    assert vrt.enc_attn_feed([st], 0, 1, P, P, P, 4, P, 0, check=False) == vrt.ERR_INVALID
    assert st.query(0) == (lim - 3, 0)
    sb = vrt.offline_scratch_bytes(d, 4)
    assert vrt.lib.vrt_enc_attn_offline(ctypes.byref(d), P, P, P, 4, lim - 3, P, P, sb, None) \
        == vrt.ERR_INVALID
    dd = vrt.dec_desc()
    ds = _state(dd, lim - 1)
    assert vrt.dec_attn_step([ds], 0, 1, P, P, P, 2, P, check=False) == vrt.ERR_INVALID


def test_set_attn_events_argument_checks():
    vrt.set_attn_events()                     # off: always accepted
    assert vrt.lib.vrt_set_attn_events(FAKE, None) == vrt.ERR_INVALID
    assert vrt.lib.vrt_set_attn_events(None, FAKE) == vrt.ERR_INVALID
    vrt.set_attn_events()


def test_single_hip_runtime_in_process():
    """libvrt and PyTorch must share one HIP runtime (a second runtime in the
    same process sees no GPU), whichever is imported first."""
    import subprocess
    import sys
    code = ("import sliding_window_cached_amd, torch\n"
            "maps = open('/proc/self/maps').read().split('\\n')\n"
            "paths = {l.split()[-1] for l in maps if 'libamdhip64' in l}\n"
            "print(len(paths)); print(sorted(paths))\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=root)
    assert r.returncode == 0, r.stderr
    assert r.stdout.split("\n")[0] == "1", r.stdout


def test_modulo_encoder_ring_host_rules():
    """ENC_MODRING (the encoder cache as a modulo ring): ring_slots must hold
    window - 1 + max_batch rows and be a multiple of 64; the planner never
    compacts and counts every frame, as the oracle's modulo-ring model does;
    the attention path is the same function of n as for the compacting ring;
    an explicit compaction is a no-op; modulo and compacting states never mix
    in one call."""
    M = vrt.ENC_MODRING
    d = vrt.enc_desc(kind=M)
    assert d.ring_slots == 1280 and vrt.desc_check(d) == vrt.OK
    assert vrt.desc_check(vrt.enc_desc(kind=M, ring_slots=1216)) == vrt.ERR_UNSUPPORTED  # < 1261
    assert vrt.desc_check(vrt.enc_desc(kind=M, ring_slots=1261)) == vrt.ERR_UNSUPPORTED  # not 64k
    assert vrt.desc_check(vrt.enc_desc(kind=M, ring_slots=1536)) == vrt.OK
    assert vrt.desc_check(vrt.enc_desc(kind=M, window=256, max_batch=64)) == vrt.OK   # 320 slots
    assert vrt.enc_desc(kind=M, window=256, max_batch=64).ring_slots == 320
    assert vrt.state_device_bytes(vrt.enc_desc(kind=M, n_layers=32)) == 32 * 2 * 20 * 1280 * 64 * 2
    rng = random.Random(1)
    for _ in range(50):
        r = DecRing(slots=1280)
        start = rng.randrange(0, 10 ** 6)
        r.reset(start)
        base, nkv = start, 0
        for _ in range(rng.randrange(1, 30)):
            n = rng.choice([1, 4, 31, 32, 512, 513, 2000])
            r.append(n)
            base, nkv, nc = vrt.ring_advance(d, base, nkv, n)
            assert nc == 0 and base == start and base + nkv == r.next_pos
    for n in (1, 4, 31, 32, 512):
        assert vrt.attn_path(d, n) == vrt.attn_path(vrt.enc_desc(), n)
    assert vrt.attn_path(vrt.enc_desc(kind=M, dtype=vrt.F32), 512) == 0
    st = _state(vrt.enc_desc(kind=M, n_layers=2), 5)
    vrt.ring_compact([st], 0, 2)                      # nothing to compact, nothing enqueued
    assert st.query(1) == (5, 0)
    ring = _state(vrt.enc_desc(n_layers=2))
    P = FAKE
    assert vrt.enc_attn_feed([st, ring], 0, 1, P, P, P, 4, P, 0, check=False) == vrt.ERR_INVALID
    lim = 2 ** 31
    top = _state(vrt.enc_desc(kind=M), lim - 3)
    assert vrt.enc_attn_feed([top], 0, 1, P, P, P, 4, P, 0, check=False) == vrt.ERR_INVALID
    with pytest.raises(vrt.VrtError):
        vrt.ring_advance(vrt.enc_desc(kind=M), lim - 3, 0, 4)


def test_block_entry_argument_checks():
    """vrt_rmsnorm / vrt_linear / vrt_enc_block_feed refuse bad arguments
    before anything is enqueued (no GPU work here)."""
    P = FAKE
    assert vrt.rmsnorm(P, 0, 1280, P, 1e-5, P, check=False) == vrt.ERR_INVALID
    assert vrt.rmsnorm(P, 4, 1284, P, 1e-5, P, check=False) == vrt.ERR_INVALID     # dim % 8
    assert vrt.rmsnorm(P, 4, 4096, P, 1e-5, P, check=False) == vrt.ERR_INVALID     # > 2048
    assert vrt.rmsnorm(P + 8, 4, 1280, P, 1e-5, P, check=False) == vrt.ERR_INVALID  # alignment
    assert vrt.rmsnorm(P, 4, 1280, P, -1.0, P, check=False) == vrt.ERR_INVALID
    assert vrt.linear(P, 4, 1280, P, 1300, None, None, P, check=False) == vrt.ERR_UNSUPPORTED
    assert vrt.linear(P, 4, 100, P, 1280, None, None, P, check=False) == vrt.ERR_UNSUPPORTED
    assert vrt.linear(P, 0, 1280, P, 1280, None, None, P, check=False) == vrt.ERR_INVALID
    assert vrt.linear(None, 4, 1280, P, 1280, None, None, P, check=False) == vrt.ERR_INVALID
    d = vrt.enc_desc()
    st = _state(d)
    bw = vrt.block_weights(P, P, P, P, P, P)
    assert vrt.block_workspace_bytes(d, 8) == 5 * 8 * 1280 * 2
    ws = vrt.block_workspace_bytes(d, 4)      # one state, 4 frames
    assert vrt.enc_block_feed([st], 0, P, 4, bw, P, P, ws - 1, check=False) == vrt.ERR_CAPACITY
    assert vrt.enc_block_feed([st], 1, P, 4, bw, P, P, ws, check=False) == vrt.ERR_INVALID   # layer
    assert vrt.enc_block_feed([st], 0, None, 4, bw, P, P, ws, check=False) == vrt.ERR_INVALID
    bad = vrt.block_weights(P, P, P, P, P, P)
    bad.reserved = 1
    assert vrt.enc_block_feed([st], 0, P, 4, bad, P, P, ws, check=False) == vrt.ERR_INVALID
    f32 = _state(vrt.enc_desc(dtype=vrt.F32))
    assert vrt.enc_block_feed([f32], 0, P, 4, bw, P, P, ws, check=False) == vrt.ERR_UNSUPPORTED
    dec = _state(vrt.dec_desc())
    assert vrt.enc_block_feed([dec], 0, P, 1, bw, P, P, ws, check=False) == vrt.ERR_INVALID
    top = _state(d, 2 ** 31 - 3)
    assert vrt.enc_block_feed([top], 0, P, 4, bw, P, P, ws, check=False) == vrt.ERR_INVALID
    assert st.query(0) == (0, 0) and top.query(0) == (2 ** 31 - 3, 0)


def test_conv_stem_host_rules():
    """Host planning of the conv stem and argument errors before any enqueue."""
    P = FAKE
    nb = vrt.conv_stem_device_bytes(128, 1280)
    assert nb == 512 + 5120
    assert vrt.conv_stem_device_bytes(100, 1280) == 0
    st = vrt.ConvStem(128, 1280, P, nb)
    assert st.query() == (0, 1)
    assert [st.out_frames(n) for n in (1, 2, 3, 8, 9)] == [0, 1, 1, 4, 4]
    with pytest.raises(vrt.VrtError) as e:
        vrt.ConvStem(128, 1280, P, nb - 1)
    assert e.value.status == vrt.ERR_CAPACITY
    with pytest.raises(vrt.VrtError) as e:
        vrt.ConvStem(96, 1280, P, nb)
    assert e.value.status == vrt.ERR_UNSUPPORTED
    cw = vrt.conv_weights(P, P, P, P)
    ws = vrt.conv_workspace_bytes(128, 1280, 2, 8)
    other = vrt.ConvStem(128, 1280, P + (1 << 20), nb)
    assert vrt.conv_stem_feed([st, st], P, 8, cw, P, P, ws, check=False) == vrt.ERR_INVALID
    assert vrt.conv_stem_feed([st, other], P, 8, cw, P, P, ws - 1, check=False) == vrt.ERR_CAPACITY
    assert vrt.conv_stem_feed([st], P, 0, cw, P, P, ws, check=False) == vrt.ERR_INVALID
    assert vrt.conv_stem_feed([st], P + 8, 8, cw, P, P, ws, check=False) == vrt.ERR_INVALID
    small = vrt.ConvStem(128, 256, P, vrt.conv_stem_device_bytes(128, 256))
    assert vrt.conv_stem_feed([st, small], P, 8, cw, P, P, ws, check=False) == vrt.ERR_INVALID
    assert st.query() == (0, 1)


def test_read_probe_argument_checks():
    P = FAKE
    assert vrt.lib.vrt_read_probe(None, 1 << 20, P, None) == vrt.ERR_INVALID
    assert vrt.lib.vrt_read_probe(P + 8, 1 << 20, P, None) == vrt.ERR_INVALID
    assert vrt.lib.vrt_read_probe(P, 8, P, None) == vrt.ERR_INVALID
    assert vrt.lib.vrt_read_probe(P, 1 << 20, None, None) == vrt.ERR_INVALID


def test_tile_stream_probe_argument_checks():
    P = FAKE
    f = vrt.lib.vrt_tile_stream_probe
    big = 1 << 40
    # buf, bytes, n_wg, heads, tiles, n_regions, region_stride, kv_off, passes, first_row, last_row, flags, sink,
    # stream
    assert f(None, big, 1, 1, 1, 1, 0, 8192, 1, 0, 63, 1, P, None) == vrt.ERR_INVALID
    assert f(P + 8, big, 1, 1, 1, 1, 0, 8192, 1, 0, 63, 1, P, None) == vrt.ERR_INVALID
    assert f(P, big, 1, 1, 1, 1, 0, 8192, 1, 0, 63, 1, None, None) == vrt.ERR_INVALID
    for n_wg, heads, tiles, n_regions, passes in ((0, 1, 1, 1, 1), (1, 0, 1, 1, 1), (1, 1, 0, 1, 1),
                                                  (1, 1, 1, 0, 1), (1, 1, 1, 1, 0)):
        assert f(P, big, n_wg, heads, tiles, n_regions, 0, 8192, passes, 0, 63, 1, P, None) == vrt.ERR_INVALID
    assert f(P, big, 1, 1, 1, 1, 8, 8192, 1, 0, 63, 1, P, None) == vrt.ERR_INVALID       # stride not 16-aligned
    assert f(P, big, 1, 1, 1, 1, 0, 8200, 1, 0, 63, 1, P, None) == vrt.ERR_INVALID       # kv_off not 16-aligned
    assert f(P, big, 1, 1, 1, 1, 0, 8192, 1, 0, 63, 2, P, None) == vrt.ERR_INVALID       # unknown flag
    for first, last in ((-1, 63), (64, 63), (0, -1), (0, 64)):                           # rows outside a tile
        assert f(P, big, 1, 1, 2, 1, 0, 16384, 1, first, last, 1, P, None) == vrt.ERR_INVALID
    assert f(P, big, 1, 1, 1, 1, 0, 8192, 1, 40, 39, 1, P, None) == vrt.ERR_INVALID      # one tile, empty rows
    # the last byte read is region 3's V half, end of tile 2: 3 * 65536 + 32768 + 3 * 8192 = 253952
    assert f(P, 253951, 1, 1, 3, 4, 65536, 32768, 1, 0, 63, 0, P, None) == vrt.ERR_INVALID


def test_lookahead_host_rules():
    """ENC_LOOKAHEAD descs: no rotation (rope_theta 0), the ring must hold
    window + F + max_batch - 1 rows (F = lookahead - 1 future frames), a
    multiple of 64; answered-query counts; the vector path only; waiting
    q rows in the state; states with different numbers of waiting queries
    never share a call."""
    d = vrt.lookahead_desc(16, 4)
    assert d.ring_slots == 576 and vrt.desc_check(d) == vrt.OK          # 16 + 3 + 512 - 1 = 530
    bad = vrt.lookahead_desc(16, 4)
    bad.rope_theta = 1.0e6
    assert vrt.desc_check(bad) == vrt.ERR_INVALID
    assert vrt.desc_check(vrt.lookahead_desc(16, 4, ring_slots=512)) == vrt.ERR_UNSUPPORTED
    assert vrt.desc_check(vrt.lookahead_desc(16, 4, ring_slots=600)) == vrt.ERR_UNSUPPORTED   # not 64k
    assert vrt.desc_check(vrt.lookahead_desc(16, 0)) == vrt.OK
    assert [vrt.attn_out_frames(d, 0, n) for n in (1, 3, 4, 10)] == [0, 0, 1, 7]
    assert [vrt.attn_out_frames(d, f, 4) for f in (1, 2, 3, 100)] == [2, 3, 4, 4]
    assert vrt.attn_out_frames(vrt.lookahead_desc(16, 1), 0, 4) == 4
    assert vrt.attn_out_frames(vrt.enc_desc(), 0, 4) == 4
    assert all(vrt.attn_path(d, n) == 0 for n in (1, 4, 64, 512))
    d3 = vrt.lookahead_desc(16, 4, n_layers=2)
    ring = 2 * 8 * 576 * 64 * 2
    assert vrt.state_device_bytes(d3) == 2 * (ring + 3 * 8 * 64 * 2)
    base, nkv, nc = vrt.ring_advance(d3, 0, 0, 10)
    assert (base, nkv, nc) == (0, 10, 0)
    mixed = vrt.enc_desc()
    mixed.lookahead = 4
    assert vrt.desc_check(mixed) == vrt.ERR_INVALID        # lookahead belongs to ENC_LOOKAHEAD only
