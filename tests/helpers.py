"""Test-side helpers: overwrite logical values of generated inputs, plant ties, and move
inputs to and from the GPU binding."""
from __future__ import annotations

import numpy as np

import oracle
from synth import Spec, make_inputs, scaled_spec, workload
from synth.generate import to_bf16_bits


def rows_of(inp, b: int, positions):
    return oracle.logical_rows(inp.block_table, inp.block_size, inp.seq_stride, b, positions)


def set_integer_exact(inp, rng, scale_pow2=True):
    """Integer-exact suite: q in {-8..8}, k in {-8..8} (exact in bf16/fp8/f32), w in
    {+-1/4, +-1/2, +-1, +-2}, fp8 scales powers of two.  Every score is then a multiple of a
    power of two small enough that any fp32 summation order gives it exactly."""
    spec = inp.spec
    qv = rng.integers(-8, 9, size=inp.q_idx.shape).astype(np.float32)
    inp.q_idx[...] = qv if spec.q_dtype == "f32" else to_bf16_bits(qv)
    inp.w[...] = rng.choice(np.array([-2, -1, -0.5, -0.25, 0.25, 0.5, 1, 2], np.float32),
                            size=inp.w.shape)
    for b in range(spec.num_seqs):
        n = spec.seq_lens[b]
        rows = rows_of(inp, b, np.arange(n))
        kv = rng.integers(-8, 9, size=(n, spec.idx_dim)).astype(np.float32)
        if spec.k_dtype == "fp8":
            inp.k_pool[rows] = oracle.encode_fp8_e4m3(kv)
            e = rng.integers(-3, 4, size=n) if scale_pow2 else np.zeros(n, np.int64)
            inp.k_scale[rows] = np.ldexp(np.float32(1), e).astype(np.float32)
        elif spec.k_dtype == "bf16":
            inp.k_pool[rows] = to_bf16_bits(kv)
        else:
            inp.k_pool[rows] = kv
    return inp


def plant_ties(inp, t: int, rng, n_interior=16, n_exterior=16, n_boundary=32, margin=None):
    """Planted tie groups for query t (a decode query seeing its whole sequence).

    1. interior: the key (and scale) of the position ranked ~K/2 is copied to n_interior
       positions ranked far below K: all copies must be selected;
    2. exterior: the position ranked ~2K is copied to n_exterior low-ranked positions: none
       may be selected;
    3. after re-ranking with the oracle, the position ranked exactly K (the last selected)
       is copied to n_boundary low-ranked positions: the group then straddles the cut and
       exactly its lowest-position member must be selected.
    Returns a dict of the groups (logical positions)."""
    spec = inp.spec
    K = spec.top_k
    V = int(inp.q_visible[t])
    b = int(inp.q_seq[t])
    margin = margin if margin is not None else min(10_000, V // 8)

    def ranking():
        r = oracle.indexer_topk_query(inp, t)
        order = oracle.topk_order(r.S32, V)
        return r, order

    r, order = ranking()
    low = order[K + margin:]                      # candidates for overwriting
    pick = rng.choice(low, size=n_interior + n_exterior + n_boundary, replace=False)
    src_int, src_ext = int(order[K // 2]), int(order[min(2 * K, V - 1)])

    def copy(src, dsts):
        rs = rows_of(inp, b, [src])[0]
        rd = rows_of(inp, b, dsts)
        inp.k_pool[rd] = inp.k_pool[rs]
        if inp.k_scale is not None:
            inp.k_scale[rd] = inp.k_scale[rs]

    g_int = np.sort(pick[:n_interior])
    g_ext = np.sort(pick[n_interior:n_interior + n_exterior])
    copy(src_int, g_int)
    copy(src_ext, g_ext)
    r, order = ranking()
    src_bnd = int(order[K - 1])
    g_bnd = np.sort(pick[n_interior + n_exterior:])
    copy(src_bnd, g_bnd)
    return {"interior": np.concatenate([[src_int], g_int]),
            "exterior": np.concatenate([[src_ext], g_ext]),
            "boundary": np.sort(np.concatenate([[src_bnd], g_bnd]))}
