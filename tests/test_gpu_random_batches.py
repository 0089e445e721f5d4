"""Seeded random batches, through the C ABI: states with random histories
(so their rings sit at different fill levels and compact at different
calls) are fed in random subsets and random layer ranges, one call per
round with a random frame count (for bf16, some rounds take the vector path
and some the matrix path), and every output and every state's metadata must
equal, bit for bit, feeding each state alone (family doc "Voxtral
Realtime", Capability Validation, Batch row: batched output identical to
serial).  The launch planner groups ragged states and picks kv heads per
workgroup from the call's size, so this checks that no grouping or head
group changes a row's arithmetic."""
import numpy as np
import pytest
import torch

import sliding_window_cached_amd as vrt

from gpu_util import DEV, Pool, host, say, stream

pytestmark = pytest.mark.gpu

H, D = 20, 64


def draw(gen, shape, tdt):
    return (torch.randn(shape, generator=gen, device=DEV) * 0.5).to(tdt)


@pytest.mark.parametrize("dtype, kind, seed", [
    (vrt.BF16, vrt.ENC_RING, 0), (vrt.BF16, vrt.ENC_RING, 1),
    (vrt.F32, vrt.ENC_RING, 2), (vrt.BF16, vrt.ENC_MODRING, 3)])
def test_random_subsets_batched_equal_serial(dtype, kind, seed):
    S, L = 6, 3
    rng = np.random.default_rng([seed, 21])
    desc = vrt.enc_desc(dtype=dtype, n_layers=L, kind=kind)
    tdt = torch.bfloat16 if dtype == vrt.BF16 else torch.float32
    starts = [int(x) for x in rng.integers(0, 1_000_000, S)]
    A, B = Pool(desc, S, starts), Pool(desc, S, starts)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(100 + seed)

    def alone(pool, i, l0, nl, q, k, v, n):
        out = torch.empty_like(q)
        vrt.enc_attn_feed([pool.states[i]], l0, nl, q, k, v, n, out, stream())
        return out

    # random histories, the same in both pools
    for i in range(S):
        h = int(rng.integers(0, 1600))
        if h:
            q, k, v = (draw(gen, (1, L, h, H, D), tdt) for _ in range(3))
            alone(A, i, 0, L, q, k, v, h)
            alone(B, i, 0, L, q, k, v, h)
    for rnd in range(10):
        m = int(rng.integers(2, S + 1))
        subset = sorted(int(x) for x in rng.choice(S, m, replace=False))
        l0 = int(rng.integers(0, L))
        nl = int(rng.integers(1, L - l0 + 1))
        n = int(rng.choice([1, 3, 4, 7, 16, 31, 32, 40, 128, 300]))
        say(f"round {rnd}: states {subset}, layers {l0}..{l0 + nl - 1}, {n} frames "
            f"(path {vrt.attn_path(desc, n)})")
        q, k, v = (draw(gen, (m, nl, n, H, D), tdt) for _ in range(3))
        out = torch.empty_like(q)
        vrt.enc_attn_feed([A.states[i] for i in subset], l0, nl, q, k, v, n, out, stream())
        for j, i in enumerate(subset):
            ref = alone(B, i, l0, nl, q[j:j + 1].contiguous(), k[j:j + 1].contiguous(),
                        v[j:j + 1].contiguous(), n)
            torch.cuda.synchronize()
            assert np.array_equal(host(out[j:j + 1]), host(ref)), (seed, rnd, i)
        for i in range(S):
            for l in range(L):
                assert A.states[i].query(l) == B.states[i].query(l), (seed, rnd, i, l)
    A.close()
    B.close()


DEC_SHAPES = {   # q heads, kv heads, head_dim, dtype, window = ring
    "32/8x128 bf16 w8192": (32, 8, 128, vrt.BF16, 8192),
    "32/8x64 bf16 w2048": (32, 8, 64, vrt.BF16, 2048),
    "16/4x64 fp32 w2048": (16, 4, 64, vrt.F32, 2048),
}


@pytest.mark.parametrize("seed, shape", [(0, "32/8x128 bf16 w8192"), (1, "32/8x128 bf16 w8192"),
                                         (2, "32/8x64 bf16 w2048"), (3, "16/4x64 fp32 w2048")])
def test_decoder_random_subsets_batched_equal_serial(seed, shape):
    """Decoder states prefilled to random contexts below the window, then
    single-token steps on random subsets and layer ranges: the batched call
    (its split-K plan takes kv heads per workgroup from the call's size)
    equals each state stepped alone, bit for bit, outputs and metadata."""
    HQ, HK, DD, dtype, win = DEC_SHAPES[shape]
    S, L = 6, 3
    tdt = torch.bfloat16 if dtype == vrt.BF16 else torch.float32
    rng = np.random.default_rng([seed, 22])
    desc = vrt.dec_desc(dtype=dtype, n_layers=L, heads_q=HQ, heads_kv=HK, head_dim=DD, window=win,
                        ring_slots=win)
    A, B = Pool(desc, S, [0] * S), Pool(desc, S, [0] * S)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(200 + seed)
    ws_bytes = vrt.dec_workspace_bytes(desc, S, L, 1)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)

    def step(pool, idx, l0, nl, q, k, v, n):
        out = torch.empty_like(q)
        vrt.dec_attn_step([pool.states[i] for i in idx], l0, nl, q, k, v, n, out, ws, ws_bytes, stream())
        torch.cuda.synchronize()
        return out

    for i in range(S):
        ctx = int(rng.integers(1, win - 92))   # 8100 at window 8192, as before
        say(f"{shape}: state {i}: prefill {ctx} tokens")
        q = draw(gen, (1, L, ctx, HQ, DD), tdt)
        k, v = (draw(gen, (1, L, ctx, HK, DD), tdt) for _ in range(2))
        step(A, [i], 0, L, q, k, v, ctx)
        step(B, [i], 0, L, q, k, v, ctx)
    for rnd in range(12):
        m = int(rng.integers(2, S + 1))
        subset = sorted(int(x) for x in rng.choice(S, m, replace=False))
        l0 = int(rng.integers(0, L))
        nl = int(rng.integers(1, L - l0 + 1))
        q = draw(gen, (m, nl, 1, HQ, DD), tdt)
        k, v = (draw(gen, (m, nl, 1, HK, DD), tdt) for _ in range(2))
        out = step(A, subset, l0, nl, q, k, v, 1)
        for j, i in enumerate(subset):
            ref = step(B, [i], l0, nl, q[j:j + 1].contiguous(), k[j:j + 1].contiguous(),
                       v[j:j + 1].contiguous(), 1)
            assert np.array_equal(host(out[j:j + 1]), host(ref)), (seed, rnd, i)
        for i in range(S):
            for l in range(L):
                assert A.states[i].query(l) == B.states[i].query(l), (seed, rnd, i, l)
    A.close()
    B.close()
