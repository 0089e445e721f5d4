"""GPU edge cases of the cached path, through the C ABI.

* more states in one call than one launch takes (the host splits them into
  launches of at most 256): bit-identical to feeding each state alone;
* the degenerate window W = 1 (each query sees only itself): every output is
  its own value row, bit for bit, on both attention paths and in fp32;
* a window wider than everything fed (W >= positions seen): the oracle's plain
  causal attention, within the gpu_util tolerances;
* the top of the position range (the last frame at 2^31 - 1, the largest
  position the library accepts): the vector path with its fused append and a
  compaction, in bf16 and fp32, and the decoder's split step past its ring's
  wrap; angles of about 2.1e9 rad (streaming plan, "Unbounded length":
  absolute positions for every frame of an unbounded stream)."""
import numpy as np
import pytest
import torch

import sliding_window_cached_amd as vrt
from oracle import attention

from gpu_util import DEV, Pool, check_close, host, run_feeds, say, seqs, stream, to_dev
from synth import qkv

pytestmark = pytest.mark.gpu
THETA = 1.0e6


def test_more_states_than_one_launch():
    S, T, H, d = 300, 12, 20, 64
    desc = vrt.enc_desc(dtype=vrt.BF16, n_layers=1)
    starts = [(37 * i) % 5000 for i in range(S)]
    q, k, v = seqs(80, S, 1, T, H, d, 0.5, vrt.BF16)
    qd, kd, vd = (to_dev(x, vrt.BF16) for x in (q, k, v))
    say(f"{S} states in one call, 4-frame feeds")
    pb = Pool(desc, S, starts)
    batched = host(run_feeds(pb, range(S), 0, 1, qd, kd, vd, [4]))
    ps = Pool(desc, S, starts)
    for s in (0, 1, 255, 256, 257, 299):
        one = host(run_feeds(ps, [s], 0, 1, qd[s:s + 1], kd[s:s + 1], vd[s:s + 1], [4]))
        assert np.array_equal(one[0], batched[s]), s
    pb.close()
    ps.close()


@pytest.mark.parametrize("dtype,sizes", [(vrt.BF16, [4]), (vrt.BF16, [64]), (vrt.F32, [5])])
def test_window_one_returns_the_values(dtype, sizes):
    T, H, d = 200, 20, 64
    desc = vrt.enc_desc(dtype=dtype, n_layers=1, window=1, ring_slots=576, max_batch=512)
    q, k, v = seqs(81, 1, 1, T, H, d, 1.0, dtype)
    qd, kd, vd = (to_dev(x, dtype) for x in (q, k, v))
    pool = Pool(desc, 1, [12345])
    say(f"window 1, feeds {sizes}, path {vrt.attn_path(desc, sizes[0])}")
    out = host(run_feeds(pool, [0], 0, 1, qd, kd, vd, sizes))[0, 0]
    assert np.array_equal(out, v[0, 0])
    pool.close()


def test_window_wider_than_the_stream():
    T, H, d, start = 300, 20, 64, 7
    desc = vrt.enc_desc(dtype=vrt.BF16, n_layers=1)
    q, k, v = seqs(82, 1, 1, T, H, d, 1.0, vrt.BF16)
    qd, kd, vd = (to_dev(x, vrt.BF16) for x in (q, k, v))
    pool = Pool(desc, 1, [start])
    out = host(run_feeds(pool, [0], 0, 1, qd, kd, vd, [4, 100, 4]))[0, 0]
    ref = attention.windowed(q[0, 0], k[0, 0], v[0, 0], start, T + 10, THETA)
    check_close(out, ref, vrt.BF16, "window wider than the stream")
    pool.close()


@pytest.mark.parametrize("dtype", [vrt.BF16, vrt.F32])
def test_vector_path_at_the_top_of_the_position_range(dtype):
    T, H, d = 1600, 20, 64
    start = 2 ** 31 - T          # the last frame is at 2^31 - 1
    desc = vrt.enc_desc(dtype=dtype, n_layers=1)
    q, k, v = seqs(83, 1, 1, T, H, d, 1.0, dtype)
    qd, kd, vd = (to_dev(x, dtype) for x in (q, k, v))
    outs = []
    for sizes in ([4], [1, 3, 2, 7]):
        pool = Pool(desc, 1, [start])
        say(f"dtype {dtype}: feeds {sizes} from position {start}")
        outs.append(host(run_feeds(pool, [0], 0, 1, qd, kd, vd, sizes))[0, 0])
        pool.close()
    assert np.array_equal(outs[0], outs[1])
    ts = [0, 1, 749, 750, 1535, 1536, 1537, T - 2, T - 1]
    ref = attention.windowed_at(q[0, 0], k[0, 0], v[0, 0], start, 750, THETA, ts)
    check_close(outs[0][ts], ref, dtype, "vector path at the top of the position range")


def test_decoder_at_the_top_of_the_position_range():
    T = 8300
    start = 2 ** 31 - T
    desc = vrt.dec_desc()
    q, k, v = qkv(84, 0, 0, T, 32, 8, 128, 1.0, "bf16")
    qd, kd, vd = (to_dev(x, vrt.BF16) for x in (q, k, v))
    pool = Pool(desc, 1, [start])
    ws_b = vrt.dec_workspace_bytes(desc, 1, 1, 1)
    ws = torch.empty(ws_b, dtype=torch.uint8, device=DEV)
    out = torch.empty_like(qd)
    say(f"decoder from position {start}: 16 x 512 prefill, then {T - 8192} single steps")
    t = 0
    for n in [512] * 16 + [1] * (T - 8192):
        o = torch.empty_like(qd[t:t + n])
        vrt.dec_attn_step(pool.states, 0, 1, qd[t:t + n].contiguous(), kd[t:t + n].contiguous(),
                          vd[t:t + n].contiguous(), n, o, ws, ws_b, stream())
        out[t:t + n] = o
        t += n
    torch.cuda.synchronize()
    pool.close()
    ts = [0, 8191, 8192, 8250, T - 1]
    ref = attention.windowed_at(q, k, v, start, 8192, THETA, ts)
    check_close(host(out)[ts], ref, vrt.BF16, "decoder at the top of the position range")
