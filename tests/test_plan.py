"""CPU tests of the launch planner (vrt_attn_plan): the key splits and query
chunks of a sub-batch depend only on the cache kind and the sub-batch size,
never on how many caches share the launch, so a state fed alone and the same
state fed in a batch take the same reductions (the pages' batch-equals-serial
check, family doc "Voxtral Realtime", Capability Validation, Batch row); the
kv heads per workgroup always divide the kv heads; and the catch-up path,
512-frame sub-batches (streaming plan, "Unbounded length"), takes the
matrix-core kernel's 128-query tiles.  Host logic only: no GPU."""
import pytest

import sliding_window_cached_amd as vrt

UNITS = [1, 2, 7, 32, 64, 256, 832, 2048, 8192]


def test_decoder_single_token_splits_the_window():
    desc = vrt.dec_desc()
    for u in UNITS:
        hg, splits, qc = vrt.attn_plan(desc, u, 1)
        # window 8192 in absolute-aligned spans of 2048 keys: 4 full spans
        # plus the one the window's ragged start falls in
        assert splits == 5 and qc == 1
        assert hg >= 1 and 8 % hg == 0


def test_decoder_prefill_is_not_split():
    desc = vrt.dec_desc()
    for n in (2, 16, 17, 511, 512):
        for u in UNITS:
            hg, splits, qc = vrt.attn_plan(desc, u, n)
            assert splits == 1
            # 16 rows per chunk: 4 query positions of a 4-head GQA group
            assert qc == -(-n // 4)
            assert 8 % hg == 0


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 16, 31])
def test_encoder_small_sub_batches_take_the_vector_path(n):
    desc = vrt.enc_desc()
    plans = {vrt.attn_plan(desc, u, n)[1:] for u in UNITS}
    # one chunk of up to 16 query rows, no key splits, whatever the unit count
    assert plans == {(1, -(-n // 16))}
    for u in UNITS:
        hg = vrt.attn_plan(desc, u, n)[0]
        assert hg >= 1 and 20 % hg == 0


@pytest.mark.parametrize("n", [32, 100, 128, 129, 300, 512])
def test_encoder_catch_up_takes_128_query_tiles(n):
    desc = vrt.enc_desc()
    for u in UNITS:
        assert vrt.attn_plan(desc, u, n) == (1, 1, -(-n // 128))


def test_matrix_path_needs_bf16_and_one_query_head_per_kv_head():
    # fp32 storage and grouped heads stay on the vector kernel at any size
    assert vrt.attn_plan(vrt.enc_desc(dtype=vrt.F32), 32, 512)[2] == 32   # 16-row chunks
    grouped = vrt.enc_desc()
    grouped.n_heads_kv = 5                                                # 4 query heads per kv head
    assert vrt.attn_plan(grouped, 32, 512)[2] == 128                      # 4 positions x 4 heads
    assert vrt.attn_plan(vrt.enc_desc(), 32, 512)[2] == 4                 # 128-query tiles


def test_lookahead_and_modulo_ring_plans_do_not_depend_on_units():
    for desc in (vrt.lookahead_desc(16, 4), vrt.lookahead_desc(16, 4, head_dim=40),
                 vrt.enc_desc(kind=vrt.ENC_MODRING)):
        for n in (1, 4, 64):
            assert len({vrt.attn_plan(desc, u, n)[1:] for u in UNITS}) == 1


def test_one_unit_alone_takes_one_kv_head_per_workgroup():
    # a single cache spreads its heads over workgroups, so it fills more CUs
    assert vrt.attn_plan(vrt.enc_desc(), 1, 4)[0] == 1
    assert vrt.attn_plan(vrt.dec_desc(), 1, 1)[0] == 1


def test_argument_errors():
    desc = vrt.enc_desc()
    for units, n in ((0, 4), (-1, 4), (1, 0), (1, -5), (1 << 41, 4)):
        with pytest.raises(vrt.VrtError):
            vrt.attn_plan(desc, units, n)
    bad = vrt.enc_desc()
    bad.head_dim = 96
    with pytest.raises(vrt.VrtError):
        vrt.attn_plan(bad, 1, 4)
