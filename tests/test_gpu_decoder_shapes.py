"""GPU parity of the decode step (split-K attention and merge) across GQA
groups, head widths and storage types.

Each split's partial record holds one 128-byte line of (m, l) for the split's
query rows, then the rows' accumulators. Group 16 fills that line: 16 q heads
per kv head, i.e. 16 rows, four per wave. Group 1 leaves one row. Head_dim 64
gives one accumulator register per lane. For each shape, a 39-token prefill
and a 20-token prefill are followed by single-token steps past the 256-slot
ring's wrap. The 256-slot ring and a 1024-slot buffer that never wraps must
give the same bits, and both must match the fp64 oracle."""
import numpy as np
import pytest
import torch

import sliding_window_cached_amd as vrt
from oracle import attention
from synth import qkv

from gpu_util import DEV, Pool, check_close, host, say, stream, to_dev

pytestmark = pytest.mark.gpu
THETA = 1.0e6
W = 256

SHAPES = [   # (q heads, kv heads, head_dim, dtype)
    (32, 2, 128, vrt.BF16),
    (32, 2, 64, vrt.F32),
    (8, 8, 64, vrt.BF16),
    (16, 4, 64, vrt.F32),
]


def _dec_run(desc, q, k, v, schedule):
    T = q.shape[0]
    pool = Pool(desc, 1, [0])
    qd, kd, vd = (to_dev(x, desc.dtype) for x in (q, k, v))
    ws_b = vrt.dec_workspace_bytes(desc, 1, 1, 1)
    ws = torch.empty(ws_b // 4 + 1, dtype=torch.float32, device=DEV)
    out = torch.empty_like(qd)
    t = 0
    for n in schedule:
        o = torch.empty_like(qd[t:t + n])
        vrt.dec_attn_step(pool.states, 0, 1, qd[t:t + n].contiguous(), kd[t:t + n].contiguous(),
                          vd[t:t + n].contiguous(), n, o, ws, ws_b, stream())
        out[t:t + n] = o
        t += n
    assert t == T
    torch.cuda.synchronize()
    res = host(out)
    pool.close()
    return res


@pytest.mark.parametrize("hq,hkv,d,dtype", SHAPES)
def test_decode_step_shapes(hq, hkv, d, dtype):
    T = 420
    q, k, v = qkv(43 + hq + d, 0, 0, T, hq, hkv, d, 1.0, "bf16" if dtype == vrt.BF16 else "f32")
    sched = [39, 20] + [1] * (T - 59)
    mk = lambda slots: vrt.dec_desc(dtype=dtype, heads_q=hq, heads_kv=hkv, head_dim=d, window=W,
                                     ring_slots=slots)
    what = f"decoder {hq}/{hkv} x {d} {'bf16' if dtype == vrt.BF16 else 'fp32'}"
    say(f"{what}: ring 256 and linear 1024")
    ring = _dec_run(mk(256), q, k, v, sched)
    lin = _dec_run(mk(1024), q, k, v, sched)
    assert np.array_equal(ring, lin), "ring and never-wrapping buffer differ"
    ref = attention.windowed(q, k, v, 0, W, THETA)
    check_close(ring, ref, dtype, what)
