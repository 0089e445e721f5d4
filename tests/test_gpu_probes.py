"""The two measurement kernels run through the C ABI: the streaming-read
probe and the tile-stream probe (the vector attention kernel's K/V tile
loop with no arithmetic).  They write nothing but, never in practice, one
word to their sink, so after a call the sink still holds zeros; the
tile-stream probe reads exactly the bytes its arguments name, and a buffer
one byte short is refused before anything is enqueued."""
import pytest
import torch

import sliding_window_cached_amd as vrt

from gpu_util import DEV, say, stream

pytestmark = pytest.mark.gpu


def test_read_probe_leaves_the_sink_alone():
    buf = torch.ones(1 << 24, dtype=torch.uint8, device=DEV)
    sink = torch.zeros(4, dtype=torch.int32, device=DEV)
    vrt.read_probe(buf, buf.numel(), sink, stream())
    torch.cuda.synchronize()
    assert sink.cpu().tolist() == [0, 0, 0, 0]


@pytest.mark.parametrize("n_wg, heads, tiles, n_regions, passes", [
    (8, 5, 12, 40, 1),        # the serving shape, scaled down: one region per (workgroup, head)
    (64, 1, 4, 16, 3),        # regions shared round robin, several passes
    (3, 2, 1, 1, 2),          # one region, one tile
])
def test_tile_stream_probe_reads_inside_its_buffer(n_wg, heads, tiles, n_regions, passes):
    stride, kv_off = 2 * tiles * 8192, tiles * 8192
    need = (n_regions - 1) * stride + kv_off + tiles * 8192
    buf = torch.ones(need, dtype=torch.uint8, device=DEV)
    sink = torch.zeros(4, dtype=torch.int32, device=DEV)
    say(f"tile stream probe: {n_wg} workgroups x {heads} heads x {tiles} tiles over {n_regions} regions "
        f"({need} bytes), {passes} passes")
    assert vrt.lib.vrt_tile_stream_probe(vrt._ptr(buf), need - 1, n_wg, heads, tiles, n_regions, stride, kv_off,
                                         passes, 0, 63, 1, vrt._ptr(sink), stream()) == vrt.ERR_INVALID
    for nt in (True, False):
        vrt.tile_stream_probe(buf, need, n_wg, heads, tiles, n_regions, stride, kv_off, passes, sink, stream(),
                              nontemporal=nt)
    # a window's edge tiles: the first read from row 32, the last up to row 16 (one tile: rows 16..32)
    first, last = (32, 16) if tiles > 1 else (16, 32)
    vrt.tile_stream_probe(buf, need, n_wg, heads, tiles, n_regions, stride, kv_off, passes, sink, stream(),
                          first_row=first, last_row=last)
    torch.cuda.synchronize()
    assert sink.cpu().tolist() == [0, 0, 0, 0]
