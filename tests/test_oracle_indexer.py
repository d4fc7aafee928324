"""Pins of the oracle's indexer scores and Top-K against a hand-worked example, exact
integer arithmetic, math.fsum loops, closed forms (one-hot head weight, power-of-two weight
scaling) and an O(V^2) brute-force rank that does not sort."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from synth import make_inputs, scaled_spec, workload
from tests.helpers import plant_ties, rows_of, set_integer_exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "indexer_worked_example.json")))
    q = np.array(g["q"], np.float64)
    w = np.array(g["w"], np.float64)
    k = np.array(g["keys"], np.float64)
    S32 = oracle.to_fp32_score(oracle.index_scores(q, w, k))
    assert S32.tolist() == g["scores"]
    assert math.copysign(1.0, S32[4]) == 1.0          # the -0 score is taken as +0
    for kk, want in g["topk"].items():
        assert oracle.topk_order(S32, int(kk)).tolist() == want


def _fsum_scores(q, w, k):
    out = []
    for s in range(k.shape[0]):
        terms = []
        for h in range(q.shape[0]):
            x = math.fsum(float(a) * float(b) for a, b in zip(q[h], k[s]))
            terms.append(float(w[h]) * max(x, 0.0))
        out.append(math.fsum(terms))
    return np.array(out)


@pytest.mark.parametrize("hi,di", [(1, 7), (3, 5), (8, 64)])
def test_scores_match_fsum_loop(hi, di):
    rng = np.random.default_rng(hi * 100 + di)
    q = oracle.decode_bf16(oracle.encode_bf16_rne(rng.standard_normal((hi, di)).astype(np.float32)))
    w = rng.standard_normal(hi)
    k = oracle.decode_bf16(oracle.encode_bf16_rne(rng.standard_normal((50, di)).astype(np.float32)))
    S = oracle.index_scores(q, w, k)
    ref = _fsum_scores(q, w, k)
    mag = np.abs(k) @ np.abs(q).T @ np.abs(w)
    assert np.all(np.abs(S - ref) <= 1e-14 * mag + 1e-300)


def test_one_hot_head_weight_is_single_head_relu():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((8, 64))
    k = rng.standard_normal((300, 64))
    for h in (0, 5):
        w = np.zeros(8)
        w[h] = 1.0
        S = oracle.index_scores(q, w, k)
        single = np.array([max(math.fsum(q[h] * k[s]), 0.0) for s in range(300)])
        assert np.allclose(S, single, rtol=1e-14, atol=1e-14)
        assert np.all(S >= 0)


def test_power_of_two_weight_scaling_is_exact():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((4, 16))
    w = rng.standard_normal(4)
    k = rng.standard_normal((500, 16))
    S32 = oracle.to_fp32_score(oracle.index_scores(q, w, k))
    for e in (-3, 5):
        S32e = oracle.to_fp32_score(oracle.index_scores(q, w * 2.0 ** e, k))
        assert np.array_equal(S32e, (S32.astype(np.float64) * 2.0 ** e).astype(np.float32))
        assert np.array_equal(oracle.topk_order(S32e, 40), oracle.topk_order(S32, 40))


def _brute_rank(S32):
    V = S32.shape[0]
    rank = np.zeros(V, np.int64)
    for s in range(V):
        for u in range(V):
            if S32[u] > S32[s] or (S32[u] == S32[s] and u < s):
                rank[s] += 1
    return rank


@pytest.mark.parametrize("seed", range(6))
def test_topk_brute_force_rank_with_ties(seed):
    rng = np.random.default_rng(seed)
    V = int(rng.integers(1, 65))
    S32 = rng.choice(np.array([-1.5, -0.0, 0.0, 0.25, 1.0, 2.0, 3.5], np.float32), size=V)
    S32 = oracle.to_fp32_score(S32.astype(np.float64))
    rank = _brute_rank(S32)
    for k in range(1, V + 1):
        sel = oracle.topk_order(S32, k)
        assert sorted(sel.tolist()) == sorted(np.nonzero(rank < k)[0].tolist())
        assert sel.tolist() == np.argsort(rank)[:k].tolist()       # rank order too
    assert oracle.topk_order(S32, 1)[0] == int(np.argmax(S32))       # first maximum
    assert sorted(oracle.topk_order(S32, V).tolist()) == list(range(V))


def _exact_scores(inp, t):
    """Exact scores (as Fractions) of query t of an integer-exact input, by integer math."""
    spec = inp.spec
    b, V = int(inp.q_seq[t]), int(inp.q_visible[t])
    q = oracle.decode(inp.q_idx[t], spec.q_dtype).astype(np.int64)
    w = [Fraction(float(x)) for x in inp.w[t]]
    rows = rows_of(inp, b, np.arange(V))
    k = oracle.decode(inp.k_pool[rows], spec.k_dtype).astype(np.int64)
    sc = [Fraction(float(x)) for x in inp.k_scale[rows]] if spec.k_dtype == "fp8" else [1] * V
    x = k @ q.T                                           # int64, exact
    out = []
    for s in range(V):
        out.append(sum(w[h] * max(int(x[s, h]), 0) for h in range(q.shape[0])) * sc[s])
    return out


@pytest.mark.parametrize("k_dtype", ["fp8", "bf16", "f32"])
def test_integer_exact_suite_scores_are_exact(k_dtype):
    base = workload(4)
    spec = scaled_spec(base, seq_lens=[700, 333], k_dtype=k_dtype, idx_heads=64, idx_dim=128,
                       top_k=100)
    inp = make_inputs(spec, seed=11, with_sfa=False)
    set_integer_exact(inp, np.random.default_rng(5))
    for t in range(spec.num_queries):
        r = oracle.indexer_topk_query(inp, t)
        exact = _exact_scores(inp, t)
        assert [Fraction(float(v)) for v in r.S32] == exact
        # selection agrees with sorting the exact values
        order = sorted(range(len(exact)), key=lambda s: (-exact[s], s))[:r.k_eff]
        assert r.idx[:r.k_eff].tolist() == order


def test_fp8_scale_enters_the_scores():
    """Doubling one token's scale doubles exactly that token's score."""
    spec = scaled_spec(workload(4), seq_lens=[256], top_k=16)
    inp = make_inputs(spec, seed=3, with_sfa=False)
    r0 = oracle.indexer_topk_query(inp, 0)
    row = rows_of(inp, 0, [17])[0]
    inp.k_scale[row] *= np.float32(2)
    r1 = oracle.indexer_topk_query(inp, 0)
    assert r1.S32[17] == np.float32(2 * float(r0.S32[17]))
    mask = np.arange(256) != 17
    assert np.array_equal(r1.S32[mask], r0.S32[mask])


def test_k_larger_than_visible_keeps_everything():
    spec = scaled_spec(workload(2), seq_lens=[50, 3000], q_seq=[0, 1, 1], q_visible=[50, 1, 2047],
                       top_k=2048)
    inp = make_inputs(spec, seed=9, with_sfa=False)
    rs = oracle.indexer_topk(inp)
    assert [r.k_eff for r in rs] == [50, 1, 2047]
    for r in rs:
        assert sorted(r.idx[:r.k_eff].tolist()) == list(range(r.k_eff))
        assert np.all(r.idx[r.k_eff:] == -1)


def test_planted_ties_have_intended_status():
    spec = scaled_spec(workload(5), seq_lens=[40000], top_k=512)
    inp = make_inputs(spec, seed=5, with_sfa=False)
    groups = plant_ties(inp, 0, np.random.default_rng(1), margin=2000)
    r = oracle.indexer_topk_query(inp, 0)
    sel = set(r.idx[:r.k_eff].tolist())
    S = r.S32
    for name, g in groups.items():
        assert len(set(S[g].tolist())) == 1, name            # bit-identical scores
    assert set(groups["interior"].tolist()) <= sel
    assert not (set(groups["exterior"].tolist()) & sel)
    bnd = groups["boundary"]
    assert [p in sel for p in bnd.tolist()] == [True] + [False] * (len(bnd) - 1)


def test_mxfp8_path_quantizes_query_and_keys():
    """With integer-exact queries and keys (lossless in MXFP8) the MXFP8 path equals the fp32
    path exactly; with general values it equals the fp32 path run on the MX-dequantized query
    and keys, which differs from the unquantized scores."""
    import dataclasses
    rng = np.random.default_rng(3)
    spec = scaled_spec(workload(1), seq_lens=[700], idx_heads=8, idx_dim=64, top_k=50)
    inp = make_inputs(spec, seed=3, with_sfa=False)
    rows = rows_of(inp, 0, np.arange(700))
    for exact in (True, False):
        kf = (rng.integers(-8, 9, (700, 64)) if exact else rng.standard_normal((700, 64))).astype(np.float32)
        qf = (rng.integers(-8, 9, inp.q_idx.shape) if exact else rng.standard_normal(inp.q_idx.shape)).astype(np.float32)
        inp.k_pool[rows] = kf
        inp.q_idx[...] = qf
        codes = np.zeros(inp.k_pool.shape, np.uint8)
        sb = np.zeros((inp.k_pool.shape[0], 2), np.uint8)
        codes[rows], sb[rows] = oracle.quantize_mxfp8(kf)
        mx = dataclasses.replace(inp, spec=dataclasses.replace(spec, k_dtype="mxfp8"),
                                 k_pool=codes, k_scale=sb)
        S_mx = oracle.indexer_topk_query(mx, 0).S32
        S_f32 = oracle.indexer_topk_query(inp, 0).S32
        if exact:
            assert np.array_equal(S_mx, S_f32)
        else:
            deq = dataclasses.replace(inp, k_pool=inp.k_pool.copy(), q_idx=inp.q_idx.copy())
            deq.k_pool[rows] = oracle.decode_mxfp8(codes[rows], sb[rows]).astype(np.float32)
            deq.q_idx[...] = oracle.decode_mxfp8(*oracle.quantize_mxfp8(qf)).astype(np.float32)
            assert np.array_equal(S_mx, oracle.indexer_topk_query(deq, 0).S32)
            assert not np.array_equal(S_mx, S_f32)
