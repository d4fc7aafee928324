"""Pins of the oracle's paged addressing: a hand-built block table, a random scatter built
here (not by the generator) that depaging must undo, and the generator's layout (every
visible row finite, every unused row NaN)."""
import numpy as np

import oracle
from synth import make_inputs, scaled_spec, workload


def test_hand_built_block_table():
    bt = np.array([[2, 0, 7], [1, 3, 7]], np.int32)      # block size 2
    rows = oracle.logical_rows(bt, 2, 0, 0, [0, 1, 2, 3])
    assert rows.tolist() == [4, 5, 0, 1]
    rows = oracle.logical_rows(bt, 2, 0, 1, [0, 1, 2, 3])
    assert rows.tolist() == [2, 3, 6, 7]
    assert oracle.logical_rows(None, 0, 100, 3, [0, 99]).tolist() == [300, 399]


def test_depage_undoes_a_random_scatter():
    rng = np.random.default_rng(0)
    bs, lens = 64, [1000, 64, 130]
    logical = [rng.standard_normal((n, 5)) for n in lens]
    nblk = [-(-n // bs) for n in lens]
    perm = rng.permutation(sum(nblk) + 3)
    bt = np.zeros((3, max(nblk)), np.int32)
    pool = np.full(((sum(nblk) + 3) * bs, 5), np.nan)
    off = 0
    for b, n in enumerate(lens):
        bt[b, :nblk[b]] = perm[off:off + nblk[b]]
        off += nblk[b]
        for s in range(n):
            pool[bt[b, s // bs] * bs + s % bs] = logical[b][s]
    for b, n in enumerate(lens):
        assert np.array_equal(oracle.depage(pool, bt, bs, 0, b, n), logical[b])


def test_generator_layout_visible_rows_finite_rest_nan():
    spec = scaled_spec(workload(4), seq_lens=[200, 64, 1], extra_blocks=3)
    inp = make_inputs(spec, seed=1)
    used = np.zeros(inp.kv_pool.shape[0], bool)
    for b, n in enumerate(spec.seq_lens):
        r = oracle.logical_rows(inp.block_table, 64, 0, b, np.arange(n))
        assert np.unique(r).size == n
        used[r] = True
        assert not np.isnan(oracle.decode(inp.kv_pool[r], "bf16")).any()
        assert not np.isnan(oracle.decode(inp.k_pool[r], "fp8")).any()
        assert not np.isnan(inp.k_scale[r]).any()
    assert np.isnan(oracle.decode(inp.kv_pool[~used], "bf16")).all()
    assert np.isnan(oracle.decode(inp.k_pool[~used], "fp8")).all()
    # spare block-table columns point at a NaN block
    spare = inp.block_table[0, -1]
    assert np.isnan(inp.k_scale[spare * 64:(spare + 1) * 64]).all()


def test_generator_is_deterministic():
    spec = scaled_spec(workload(2), seq_lens=[100, 300], sfa_heads=4)
    a, b = make_inputs(spec, seed=3), make_inputs(spec, seed=3)
    for f in ("q_idx", "w", "k_pool", "q_sfa", "kv_pool", "block_table"):
        assert np.array_equal(getattr(a, f), getattr(b, f), equal_nan=False) or \
            np.array_equal(getattr(a, f).view(np.uint8), getattr(b, f).view(np.uint8))
    c = make_inputs(spec, seed=4)
    assert not np.array_equal(a.q_idx, c.q_idx)
