"""GPU parity of dsa_indexer_topk against the oracle, through the C ABI.

Tolerance (per query): the returned set has exactly K_eff distinct positions in [0, V) and
differs from the oracle's only at positions whose fp32 score is within 1e-6 relative of the
oracle's K-th score.  Strict suites (integer-exact scores, planted ties between
bit-identical keys, the fp8 code table) require identical sets and exact scores."""
import zlib

import numpy as np
import pytest

import oracle
from synth import make_inputs, scaled_spec, workload
from synth.device import to_device
from tests.gpu_util import log, run_indexer, score_error
from tests.helpers import plant_ties, rows_of, set_integer_exact

pytestmark = pytest.mark.gpu


def check(inp, idx, score, strict=False, queries=None, score_tol=2e-6):
    refs = oracle.indexer_topk(inp, queries)
    res = oracle.check_topk(idx, refs, strict=strict)
    errs = [score_error(score[r.t], idx[r.t], r) for r in refs]
    log(f"  {inp.spec.name}: {len(refs)} queries, in-band diffs {res.n_in_band_diff}, "
        f"max score err / kth {max(errs):.2e}")
    assert res.ok, "\n".join(res.msgs[:10])
    assert max(errs) <= score_tol
    return refs


CASES = {
    # reference path: fp32 q/k, 8 heads x 64, contiguous, K=256 (the tiny workload, full size)
    "tiny_fp32": lambda: workload(1),
    "tiny_fp32_paged": lambda: scaled_spec(workload(1), seq_lens=[4096, 1500, 33], block_size=16,
                                           permute=True, extra_blocks=2),
    # MFMA path, bf16 keys: lengths around K and the 64-token pages, several splits
    "bf16_mixed": lambda: scaled_spec(workload(2), seq_lens=[5000, 777, 9000, 64, 1, 130, 2047,
                                                             2048, 2049, 63, 65]),
    "bf16_k100": lambda: scaled_spec(workload(2), seq_lens=[5000, 9000, 130, 17000], top_k=100),
    "bf16_bs128": lambda: scaled_spec(workload(2), seq_lens=[12345, 3000], block_size=128),
    # smallest page size of the MFMA path: every 32-position group is one whole page
    "bf16_bs32": lambda: scaled_spec(workload(2), seq_lens=[4100, 2000, 31], block_size=32),
    "fp8_bs32": lambda: scaled_spec(workload(4), seq_lens=[9000, 33], block_size=32),
    # MFMA path, fp8 keys with per-token scales
    "fp8_mixed": lambda: scaled_spec(workload(4), seq_lens=[20000, 3333, 2049, 65, 1]),
    "fp8_k256": lambda: scaled_spec(workload(4), seq_lens=[30000, 70000], top_k=256),
    # 65..255 queries: the rectangular launch even with the host's total (no compact, no tiles)
    "bf16_T100_ragged": lambda: scaled_spec(workload(2), seq_lens=[int(x) for x in
                                            np.random.default_rng(100).integers(1, 9000, 100)]),
    "fp8_T200_ragged": lambda: scaled_spec(workload(4), seq_lens=[int(x) for x in
                                           np.random.default_rng(200).integers(1, 5000, 200)]),
    # degenerate Top-K sizes on the fast path: K = 1, and K >= V (every position selected)
    "fp8_k1": lambda: scaled_spec(workload(4), seq_lens=[5000, 1, 70, 2049], top_k=1),
    "bf16_k_all": lambda: scaled_spec(workload(2), seq_lens=[100, 2048, 700, 1]),
    # reference path with mixed formats
    "ref_bf16q_fp8k": lambda: scaled_spec(workload(4), seq_lens=[3000, 5000], idx_heads=16,
                                          idx_dim=64, top_k=300),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_indexer_matches_oracle(dsa, case):
    spec = CASES[case]()
    inp = make_inputs(spec, seed=zlib.crc32(case.encode()) % 1000, with_sfa=False)
    log(f"case {case}: T={spec.num_queries} maxV={spec.max_visible} K={spec.top_k}")
    idx, score = run_indexer(dsa, inp)
    check(inp, idx, score, score_tol=2e-6 if spec.idx_heads == 64 else 1e-6)


@pytest.mark.parametrize("k_dtype", ["bf16", "fp8"])
def test_integer_exact_suite_is_bit_exact(dsa, k_dtype):
    spec = scaled_spec(workload(4), seq_lens=[6000, 1500, 64, 65, 20000], k_dtype=k_dtype,
                       top_k=512)
    inp = make_inputs(spec, seed=21, with_sfa=False)
    set_integer_exact(inp, np.random.default_rng(3))
    idx, score = run_indexer(dsa, inp)
    refs = check(inp, idx, score, strict=True, score_tol=0.0)
    for r in refs:
        assert np.array_equal(score[r.t][:r.k_eff], r.S32[idx[r.t][:r.k_eff]])


def test_fp8_code_table_through_the_fast_path(dsa):
    """Each key holds one fp8 code in dim 77 (scale 1); head 0 of the query is +-e_77 and the
    only weighted head, so every score is ReLU(+-code value): all 254 finite codes come
    back exactly through the MFMA path's fp8 widening."""
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    V = codes.size
    spec = scaled_spec(workload(4), seq_lens=[V], q_seq=[0, 0], q_visible=[V, V], top_k=V)
    inp = make_inputs(spec, seed=2, with_sfa=False)
    rows = rows_of(inp, 0, np.arange(V))
    inp.k_pool[rows] = 0
    inp.k_pool[rows, 77] = codes
    inp.k_scale[rows] = 1.0
    inp.q_idx[...] = 0
    inp.q_idx[0, 0, 77] = 0x3F80          # +1.0 (bf16 bits)
    inp.q_idx[1, 0, 77] = 0xBF80          # -1.0
    inp.w[...] = 0
    inp.w[:, 0] = 1.0
    idx, score = run_indexer(dsa, inp)
    vals = oracle.decode_fp8_e4m3(codes)
    for t, sign in ((0, 1.0), (1, -1.0)):
        got = np.zeros(V)
        got[idx[t]] = score[t]
        assert np.array_equal(got, np.maximum(sign * vals, 0.0)), t
    check(inp, idx, score, strict=True, score_tol=0.0)


def test_planted_ties_select_lowest_position(dsa):
    spec = scaled_spec(workload(5), seq_lens=[200000], top_k=2048)
    inp = make_inputs(spec, seed=55, with_sfa=False)
    groups = plant_ties(inp, 0, np.random.default_rng(7))
    idx, score = run_indexer(dsa, inp)
    refs = check(inp, idx, score)
    sel = set(idx[0][:refs[0].k_eff].tolist())
    assert set(groups["interior"].tolist()) <= sel
    assert not (set(groups["exterior"].tolist()) & sel)
    bnd = groups["boundary"]
    assert [p in sel for p in bnd.tolist()] == [True] + [False] * (len(bnd) - 1)
    assert len(set(score[0][np.isin(idx[0], groups["interior"])].tolist())) == 1


def test_concentrated_top_positions_take_the_fallback(dsa):
    """All of the top positions sit in one stretch of the context, far more than any split's
    share, so split thresholds cut too high and the merge must re-score those splits."""
    spec = scaled_spec(workload(2), seq_lens=[40000, 30000], top_k=1500)
    inp = make_inputs(spec, seed=77, with_sfa=False)
    for b, (lo, hi) in enumerate([(8000, 10000), (29000, 30000)]):
        rows = rows_of(inp, b, np.arange(lo, hi))
        k = oracle.decode_bf16(inp.k_pool[rows]) * 4.0          # exact in bf16
        inp.k_pool[rows] = oracle.encode_bf16_rne(k.astype(np.float32))
    idx, score = run_indexer(dsa, inp)
    check(inp, idx, score)


def test_layout_invariance_and_determinism(dsa):
    spec = scaled_spec(workload(4), seq_lens=[30000, 9000])
    paged = make_inputs(spec, seed=5, with_sfa=False)
    contig_spec = scaled_spec(spec, block_size=0, permute=False, extra_blocks=0)
    contig = make_inputs(contig_spec, seed=5, with_sfa=False)
    stride = contig.seq_stride
    for b, n in enumerate(spec.seq_lens):
        r = rows_of(paged, b, np.arange(n))
        contig.k_pool[b * stride:b * stride + n] = paged.k_pool[r]
        contig.k_scale[b * stride:b * stride + n] = paged.k_scale[r]
    contig.q_idx[...] = paged.q_idx
    contig.w[...] = paged.w
    i1, s1 = run_indexer(dsa, paged)
    i2, s2 = run_indexer(dsa, paged)
    i3, s3 = run_indexer(dsa, contig)
    assert np.array_equal(i1, i2) and np.array_equal(s1.view(np.uint32), s2.view(np.uint32))
    assert np.array_equal(i1, i3) and np.array_equal(s1.view(np.uint32), s3.view(np.uint32))


def test_total_visible_hint_changes_the_launch_not_the_result(dsa):
    """The host hint only picks the split length: no hint, the true total, one far too small
    and one far too large give bit-identical outputs (every position's score is summed the
    same way whatever split holds it, and the output is in position order)."""
    spec = scaled_spec(workload(4), seq_lens=[70000, 9000, 120000, 2100])
    inp = make_inputs(spec, seed=12, with_sfa=False)
    d = to_device(inp)
    ws = dsa.zeroed_workspace(dsa.indexer_workspace_bytes(spec.num_queries, d.max_visible,
                                                          spec.top_k), "cuda")
    outs = [run_indexer(dsa, inp, d, workspace=ws, total_visible=tv)
            for tv in ("exact", 0, 1, 10 ** 12)]
    check(inp, outs[0][0], outs[0][1])
    for i, s in outs[1:]:
        assert np.array_equal(i, outs[0][0])
        assert np.array_equal(s.view(np.uint32), outs[0][1].view(np.uint32))


def test_workspace_reuse_across_sizes(dsa):
    """One zero-initialised workspace serves a large call and then smaller ones."""
    big = scaled_spec(workload(2), seq_lens=[40000, 40000, 3000])
    small = scaled_spec(workload(2), seq_lens=[9000])
    inp_b = make_inputs(big, seed=1, with_sfa=False)
    inp_s = make_inputs(small, seed=2, with_sfa=False)
    ws = dsa.zeroed_workspace(dsa.indexer_workspace_bytes(3, 40000, 2048), "cuda")
    for inp in (inp_b, inp_s, inp_b):
        idx, score = run_indexer(dsa, inp, workspace=ws)
        check(inp, idx, score)


def test_workspace_reuse_from_few_to_many_queries(dsa):
    """A call with few queries, then one with more than 64 on the same workspace: the first
    call's split headers must not land on the second call's arrival counters (the counters
    keep a block of their own at the workspace's start, zero between calls)."""
    few = scaled_spec(workload(2), seq_lens=[40000, 40000, 3000])
    many = scaled_spec(workload(2), seq_lens=[int(x) for x in
                                              np.random.default_rng(101).integers(2100, 9000, 100)])
    inp_f = make_inputs(few, seed=3, with_sfa=False)
    inp_m = make_inputs(many, seed=4, with_sfa=False)
    ws = dsa.zeroed_workspace(dsa.indexer_workspace_bytes(100, 40000, 2048), "cuda")
    for inp in (inp_f, inp_m, inp_f, inp_m):
        idx, score = run_indexer(dsa, inp, workspace=ws)
        check(inp, idx, score)


# ---- full-size workloads (all queries, or a sample the oracle can score) ---------------------
@pytest.mark.slow
def test_full_decode_bf16_32k(dsa):
    inp = make_inputs(workload(2), seed=2, with_sfa=False)
    idx, score = run_indexer(dsa, inp)
    check(inp, idx, score)


@pytest.mark.slow
def test_full_decode_fp8_128k(dsa):
    inp = make_inputs(workload(4), seed=4, with_sfa=False)
    idx, score = run_indexer(dsa, inp)
    check(inp, idx, score)


@pytest.mark.slow
def test_full_decode_fp8_1m_with_planted_ties(dsa):
    inp = make_inputs(workload(5), seed=5, with_sfa=False)
    groups = plant_ties(inp, 0, np.random.default_rng(5))
    idx, score = run_indexer(dsa, inp)
    check(inp, idx, score)
    sel = set(idx[0][:2048].tolist())
    assert set(groups["interior"].tolist()) <= sel
    assert not (set(groups["exterior"].tolist()) & sel)
    bnd = groups["boundary"]
    assert [p in sel for p in bnd.tolist()] == [True] + [False] * (len(bnd) - 1)


def prefill_sample(T, n=64):
    """n evenly spaced queries of a chunk, shifted so that every position inside a four-query
    tile occurs (query 64i + i % 4), plus the last query."""
    step = T // n
    return sorted({step * i + i % 4 for i in range(n)} | {T - 1})


def check_structure(inp, idx):
    """Cheap invariants of every row: K_eff strictly increasing positions in [0, V) (the output
    is in ascending position order), then -1."""
    K = inp.spec.top_k
    for t in range(inp.spec.num_queries):
        V = int(inp.q_visible[t])
        k = min(K, V)
        head, tail = idx[t, :k], idx[t, k:]
        assert np.all(tail == -1), f"query {t}: tail not -1"
        assert head[0] >= 0 and head[-1] < V, f"query {t}: positions outside [0, {V})"
        assert np.all(np.diff(head) > 0), f"query {t}: not strictly increasing"


@pytest.mark.slow
def test_full_chunked_prefill_sampled(dsa):
    inp = make_inputs(workload(3), seed=3, with_sfa=False)
    idx, score = run_indexer(dsa, inp)
    check_structure(inp, idx)
    check(inp, idx, score, queries=prefill_sample(inp.spec.num_queries))


@pytest.mark.slow
def test_max_context_single_query(dsa):
    """The longest context a query may have (DSA_MAX_CONTEXT = 4M positions): 2048 splits of
    2048 positions, the most a query can have, all merged by one workgroup."""
    spec = scaled_spec(workload(5), seq_lens=[1 << 22])
    inp = make_inputs(spec, seed=22, with_sfa=False)
    idx, score = run_indexer(dsa, inp)
    check(inp, idx, score)
