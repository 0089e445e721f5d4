"""Seeded random start positions across the whole accepted range, through
the C ABI, against the fp64 oracle: each stream starts at a random absolute
position p0 in [0, 2^31 - T] (RoPE angles up to about 2.1e9 rad; the
streaming plan's "Unbounded length": absolute positions for every frame),
is fed on the vector path (4-frame feeds, fp32 and bf16) and on the matrix
path (512-frame feeds, bf16) across compactions, and randomly drawn rows of
every layer are checked against oracle.attention.windowed_at within the
gpu_util bounds (fp32: 1e-5 norm-wise relative; bf16: 2e-2 absolute and
1e-2 relative)."""
import numpy as np
import pytest

import sliding_window_cached_amd as vrt
from oracle import attention

from gpu_util import Pool, check_close, host, run_feeds, say, seqs, to_dev

pytestmark = pytest.mark.gpu
THETA = 1.0e6
W = 750


@pytest.mark.parametrize("dtype, sizes, seed", [
    (vrt.F32, [4], 0), (vrt.F32, [4], 1),
    (vrt.BF16, [4], 2), (vrt.BF16, [4], 3),
    (vrt.BF16, [512], 4), (vrt.BF16, [512], 5)])
def test_random_positions_against_the_oracle(dtype, sizes, seed):
    S, L, T, H, d = 3, 2, 1700, 20, 64
    rng = np.random.default_rng([seed, 31])
    starts = [int(x) for x in rng.integers(0, 2 ** 31 - T + 1, S)]
    desc = vrt.enc_desc(dtype=dtype, n_layers=L)
    scale = 0.5 if (dtype == vrt.BF16 and sizes == [4]) else 1.0
    q, k, v = seqs(110 + seed, S, L, T, H, d, scale, dtype)
    qd, kd, vd = (to_dev(x, dtype) for x in (q, k, v))
    pool = Pool(desc, S, starts)
    say(f"random starts {starts}, feeds {sizes}, {'bf16' if dtype == vrt.BF16 else 'fp32'}")
    out = host(run_feeds(pool, range(S), 0, L, qd, kd, vd, sizes))
    pool.close()
    for s in range(S):
        for l in range(L):
            ts = sorted(int(x) for x in rng.choice(T, 12, replace=False))
            ref = attention.windowed_at(q[s, l], k[s, l], v[s, l], starts[s], W, THETA, ts)
            check_close(out[s, l][ts], ref, dtype, f"start {starts[s]} layer {l} rows {ts[:4]}...")
