"""GPU test of the allocation-free decode step (vrt_dec_attn_step_static):
its split-K partials live in the library's static device array instead of a
caller workspace.  Two calls in a row, the second with fewer states and
layers than the first (so a stale partial of the first call would show),
each against vrt_dec_attn_step with a caller workspace on identically filled
caches: outputs bit-identical (same kernels, same arithmetic), ring metadata
equal.  Then the static step's outputs against the fp64 oracle on sampled
states, within the bf16 bar."""
import numpy as np
import pytest
import torch

import sliding_window_cached_amd as vrt
from oracle import attention

from gpu_util import DEV, check_close, say, stream

pytestmark = pytest.mark.gpu
THETA = 1.0e6
HQ, HK, DD, WIN = 32, 8, 128, 8192


def randn(gen, shape):
    return torch.randn(shape, generator=gen, device=DEV, dtype=torch.float32).to(torch.bfloat16)


def _fill(states, q, k, v, ctx, ws, wsb):
    """Bring state i to ctx[i] tokens: a 39-token prefill, then prefills of up
    to 512 tokens (a last chunk of one token is a decode step, with the
    caller workspace)."""
    for i, st in enumerate(states):
        t = 0
        for m in [39] + [512] * 16:
            m = min(m, ctx[i] - t)
            if m <= 0:
                break
            xs = [x[i:i + 1, :, t:t + m].contiguous() for x in (q, k, v)]
            o = torch.empty_like(xs[0])
            vrt.dec_attn_step([st], 0, q.shape[1], *xs, m, o, ws, wsb, stream())
            t += m


@pytest.mark.parametrize("seed", [50])
def test_static_decode_step_equals_workspace_step(seed):
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    results = []
    for S, L, ctx in [(8, 4, [39, 700, 1024, 1025, 3001, 5000, 8191, 8192]),
                      (3, 2, [40, 2048, 6000])]:
        desc = vrt.dec_desc(dtype=vrt.BF16, n_layers=L)
        T = max(ctx) + 1
        q = randn(gen, (S, L, T, HQ, DD))
        k = randn(gen, (S, L, T, HK, DD))
        v = randn(gen, (S, L, T, HK, DD))
        nb = vrt.state_device_bytes(desc)
        wsb = vrt.dec_workspace_bytes(desc, S, L, 1)
        ws = torch.empty(wsb // 4 + 1, dtype=torch.float32, device=DEV)
        pools = []
        for _ in range(2):
            mem = torch.empty(S * nb, dtype=torch.uint8, device=DEV)
            pools.append((mem, [vrt.StreamState(desc, mem[i * nb:(i + 1) * nb], nb, 0) for i in range(S)]))
            _fill(pools[-1][1], q, k, v, ctx, ws, wsb)
        xs = [torch.stack([x[i, :, ctx[i]:ctx[i] + 1] for i in range(S)]).contiguous() for x in (q, k, v)]
        out_ws = torch.empty((S, L, 1, HQ, DD), dtype=torch.bfloat16, device=DEV)
        out_st = torch.empty_like(out_ws)
        say(f"decode step, {S} states x {L} layers: with a workspace and allocation-free")
        vrt.dec_attn_step(pools[0][1], 0, L, *xs, 1, out_ws, ws, wsb, stream())
        vrt.dec_attn_step_static(pools[1][1], 0, L, *xs, 1, out_st, stream())
        torch.cuda.synchronize()
        a, b = out_ws.float().cpu().numpy(), out_st.float().cpu().numpy()
        assert np.isfinite(b).all()
        assert np.array_equal(a, b), (S, L)
        for i in range(S):
            assert pools[0][1][i].query(L - 1) == pools[1][1][i].query(L - 1) == (0, ctx[i] + 1)
        results.append((S, L, ctx, q, k, v, b))
        for _, states in pools:
            for st in states:
                st.close()
    # the static step against the oracle, one sampled (state, layer) per call
    for S, L, ctx, q, k, v, b in results:
        i, l = S - 1, L - 1
        t = ctx[i]
        lo = max(0, t - WIN + 1)
        ref = attention.windowed_at(*(x[i, l, lo:t + 1].float().cpu().numpy() for x in (q, k, v)), lo, WIN,
                                    THETA, [t - lo])
        check_close(b[i, l, 0], ref[0], vrt.BF16, f"static step, state {i} ctx {t}")


def test_static_decode_step_capacity_limit():
    """More partials than the static array holds: refused, nothing enqueued."""
    L = 26
    desc = vrt.dec_desc(dtype=vrt.BF16, n_layers=L)
    per_state = vrt.dec_workspace_bytes(desc, 1, L, 1)
    S = (128 << 20) // per_state + 1
    states = [vrt.StreamState(desc, 1 << 40, vrt.state_device_bytes(desc), 0) for _ in range(S)]
    s = vrt.dec_attn_step_static(states, 0, L, 1 << 41, 1 << 41, 1 << 41, 1, 1 << 41, stream(), check=False)
    assert s == vrt.ERR_CAPACITY
    assert all(st.query(0) == (0, 0) for st in states)
