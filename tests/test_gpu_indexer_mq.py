"""GPU parity of the indexer's multi-query workgroups (many queries with bf16 or fp8 keys, as
in a chunked prefill: four queries of one sequence scored together over each split), through
the C ABI.  Same tolerance as the single-query suites; and the multi-query launch must give
bit-identical results to the single-query one (DSA_INDEXER_MQ=0), since every score is the
same MFMA sum whichever workgroup computes it."""
import os

import numpy as np
import pytest

import oracle
from synth import make_inputs, scaled_spec, workload
from synth.configs import Spec
from synth.device import to_device
from tests.gpu_util import log, run_indexer, score_error
from tests.helpers import rows_of

pytestmark = pytest.mark.gpu


def chunk(L, P, **kw):
    return Spec(name=f"chunk_{P}_{L}", seq_lens=(P + L,), q_seq=(0,) * L,
                q_visible=tuple(P + i + 1 for i in range(L)), **kw)


def mixed(n_seqs, per_seq, lens, **kw):
    """Queries interleaved over sequences (q_seq = i % n_seqs), so tiles mix sequences."""
    q_seq, q_vis = [], []
    for i in range(n_seqs * per_seq):
        b = i % n_seqs
        q_seq.append(b)
        q_vis.append(max(1, lens[b] - (i // n_seqs) * 3))
    return Spec(name="mixed", seq_lens=tuple(lens), q_seq=tuple(q_seq), q_visible=tuple(q_vis))


CASES = {
    "causal_chunk_600": lambda: chunk(600, 3000),
    "causal_no_prefix_1031": lambda: chunk(1031, 0),          # ragged last tile, V < K early
    "ragged_257_k300": lambda: chunk(257, 9000, top_k=300),
    "contiguous_chunk": lambda: chunk(300, 5000, block_size=0, permute=False, extra_blocks=0),
    "bs32_chunk": lambda: chunk(280, 4100, block_size=32),
    "mixed_sequences": lambda: mixed(7, 40, [5000, 3000, 8000, 700, 64, 2049, 4500]),
    # fp8 keys with per-token scales (the quantized prefill path)
    "fp8_causal_chunk_600": lambda: chunk(600, 7000, k_dtype="fp8", k_std=1.0),
    "fp8_no_prefix_523": lambda: chunk(523, 0, k_dtype="fp8", k_std=1.0),
    "fp8_bs32_chunk": lambda: chunk(300, 3000, k_dtype="fp8", k_std=1.0, block_size=32),
    "fp8_contiguous_chunk": lambda: chunk(260, 4000, k_dtype="fp8", k_std=1.0, block_size=0,
                                          permute=False, extra_blocks=0),
}


def check(inp, idx, score, queries=None):
    refs = oracle.indexer_topk(inp, queries)
    res = oracle.check_topk(idx, refs)
    errs = [score_error(score[r.t], idx[r.t], r) for r in refs]
    log(f"  {inp.spec.name}: {len(refs)} queries checked, max score err {max(errs):.2e}")
    assert res.ok, "\n".join(res.msgs[:10])
    assert max(errs) <= 2e-6


def run_both(dsa, inp):
    d = to_device(inp)
    i1, s1 = run_indexer(dsa, inp, d)
    os.environ["DSA_INDEXER_MQ"] = "0"
    try:
        i0, s0 = run_indexer(dsa, inp, d)
    finally:
        del os.environ["DSA_INDEXER_MQ"]
    assert np.array_equal(i1, i0)
    assert np.array_equal(s1.view(np.uint32), s0.view(np.uint32))
    return i1, s1


@pytest.mark.parametrize("case", sorted(CASES))
def test_multi_query_matches_oracle_and_single_query(dsa, case):
    spec = CASES[case]()
    assert spec.num_queries >= 256
    inp = make_inputs(spec, seed=len(case) * 13, with_sfa=False)
    idx, score = run_both(dsa, inp)
    T = spec.num_queries
    sample = sorted(set(range(0, T, max(1, T // 40))) | {T - 1, T - 2, T - 3})
    check(inp, idx, score, sample)


def test_multi_query_fallback(dsa):
    """The top positions of a chunk's sequence sit in one stretch, so the splits' thresholds
    cut too high and the merges re-score splits (single-query path) after a multi-query
    scoring."""
    spec = chunk(300, 30000, top_k=1500)
    inp = make_inputs(spec, seed=78, with_sfa=False)
    rows = rows_of(inp, 0, np.arange(8000, 10000))
    k = oracle.decode_bf16(inp.k_pool[rows]) * 4.0
    inp.k_pool[rows] = oracle.encode_bf16_rne(k.astype(np.float32))
    idx, score = run_both(dsa, inp)
    check(inp, idx, score, [0, 1, 2, 3, 150, 299])


MX_CASES = {
    "mx_causal_chunk_600": lambda: chunk(600, 7000, k_dtype="f32", k_std=1.0),
    "mx_no_prefix_523": lambda: chunk(523, 0, k_dtype="f32", k_std=1.0),
}


@pytest.mark.parametrize("case", sorted(MX_CASES))
def test_multi_query_mxfp8(dsa, case):
    """MXFP8 keys (the oracle's quantization of the same fp32 keys) and queries quantized
    inside the call, per workgroup for the tile's four queries."""
    import dataclasses
    spec = MX_CASES[case]()
    inp = make_inputs(spec, seed=len(case) * 17, with_sfa=False)
    with np.errstate(invalid="ignore"):
        codes, sb = oracle.quantize_mxfp8(inp.k_pool)
    inp = dataclasses.replace(inp, spec=dataclasses.replace(spec, k_dtype="mxfp8"),
                              k_pool=codes, k_scale=sb)
    idx, score = run_both(dsa, inp)
    T = spec.num_queries
    check(inp, idx, score, sorted(set(range(0, T, max(1, T // 30))) | {T - 1}))
