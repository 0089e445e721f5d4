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


def test_decode_step_group16_two_heads_per_workgroup():
    """64 states x 8 layers of a 32/2 x 64 bf16 decoder (GQA group 16, 16
    rows per kv head, four per wave): one batched decode step, which the
    planner gives 2 kv heads per workgroup, equals the same step made state
    by state (1 kv head per workgroup) bit for bit; sampled outputs match the
    oracle."""
    S, L, HQ, HK, DD, win = 64, 8, 32, 2, 64, 2048
    desc = vrt.dec_desc(dtype=vrt.BF16, n_layers=L, heads_q=HQ, heads_kv=HK, head_dim=DD, window=win,
                        ring_slots=win)
    assert vrt.attn_plan(desc, S * L, 1)[0] == 2 and vrt.attn_plan(desc, L, 1)[0] == 1
    rng = np.random.default_rng(44)
    ctx = [int(c) for c in rng.integers(2, 300, S)]   # a prefill has 2 or more tokens
    seqs = [qkv(500 + i, i, 0, (c + 1) * L, HQ, HK, DD, 1.0, "bf16") for i, c in enumerate(ctx)]
    # per state: [L][c + 1][heads][d], token c is the decode step
    seqs = [tuple(x.reshape(L, c + 1, x.shape[1], DD) for x in s) for s, c in zip(seqs, ctx)]
    A, B = Pool(desc, S, [0] * S), Pool(desc, S, [0] * S)
    ws_b = vrt.dec_workspace_bytes(desc, S, L, 1)
    ws = torch.empty(ws_b // 4 + 1, dtype=torch.float32, device=DEV)
    say(f"group 16: prefill {S} states x {L} layers to contexts {min(ctx)}..{max(ctx)}")
    for i, c in enumerate(ctx):
        q, k, v = (to_dev(x[:, :c][None], vrt.BF16) for x in seqs[i])
        for pool in (A, B):
            o = torch.empty_like(q)
            vrt.dec_attn_step([pool.states[i]], 0, L, q, k, v, c, o, None, 0, stream())
    qs, ks, vs = (torch.stack([to_dev(s[t][:, c:c + 1], vrt.BF16) for s, c in zip(seqs, ctx)])
                  for t in range(3))
    out = torch.empty_like(qs)
    vrt.dec_attn_step(A.states, 0, L, qs, ks, vs, 1, out, ws, ws_b, stream())
    torch.cuda.synchronize()
    batched = host(out)
    for i in range(S):
        o = torch.empty_like(qs[i:i + 1])
        vrt.dec_attn_step([B.states[i]], 0, L, qs[i:i + 1].contiguous(), ks[i:i + 1].contiguous(),
                          vs[i:i + 1].contiguous(), 1, o, ws, ws_b, stream())
        torch.cuda.synchronize()
        assert np.array_equal(host(o)[0], batched[i]), ("state", i)
    for i in range(0, S, 9):
        for l in (0, L - 1):
            q, k, v = (x[l] for x in seqs[i])
            ref = attention.windowed_at(q, k, v, 0, win, THETA, [ctx[i]])
            check_close(batched[i, l, 0][None], ref, vrt.BF16, f"group 16 state {i} layer {l}")
    A.close()
    B.close()
