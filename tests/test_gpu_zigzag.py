"""GPU parity of zigzag sharding of a causal chunk, through the C ABI.

Each shard's queries (the two token ranges dsa_zigzag_ranges gives) run through
dsa_indexer_topk and dsa_sparse_attn on their own, as one device's share at its real shape,
and the rows are put back in token order.  The indexer's rows must equal the unsharded run
bit for bit (a query's selection and scores depend only on its own row and the cache).  The
attention rows must agree within the bf16 bound: a shard with few queries splits each index
list over slices merged from fp16 partials, which rounds differently from one whole pass.
Sampled queries are checked against the oracle."""
import numpy as np
import pytest

import oracle
from synth import make_inputs
from synth.configs import Spec
from synth.device import to_device
from tests.gpu_util import layout_of, log

pytestmark = pytest.mark.gpu

TOL_O, TOL_LSE = 2e-2, 1e-4


def chunk_spec(L, P):
    return Spec(name=f"chunk_{P}_{L}", seq_lens=(P + L,), q_seq=(0,) * L,
                q_visible=tuple(P + i + 1 for i in range(L)))


def run_rows(dsa, inp, d, rows):
    import torch
    spec = inp.spec
    o = torch.from_numpy(np.ascontiguousarray(rows)).cuda()
    sub = lambda x: x[o].contiguous()
    V = np.asarray(inp.q_visible)[rows]
    lay = layout_of(dsa, d)
    idx, score = dsa.indexer_topk(sub(d.q_idx), sub(d.w), d.k_pool, d.k_scale, lay, sub(d.q_seq),
                                  sub(d.q_visible), int(V.max()), spec.top_k,
                                  total_visible=int(V.sum()))
    out, lse = dsa.sparse_attn(sub(d.q_sfa), d.kv_pool, idx, lay, sub(d.q_seq),
                               spec.softmax_scale, spec.d_v)
    torch.cuda.synchronize()
    return (idx.cpu().numpy().astype(np.int64), score.cpu().numpy(),
            out.view(torch.int16).cpu().numpy(), lse.cpu().numpy())


@pytest.mark.parametrize("L,P,G", [(2500, 3000, 3), (4096, 0, 4), (777, 5000, 8)])
def test_zigzag_shards_reassemble_to_the_unsharded_result(dsa, L, P, G):
    spec = chunk_spec(L, P)
    inp = make_inputs(spec, seed=L + G, sfa_dist="sharp")
    d = to_device(inp)
    whole = run_rows(dsa, inp, d, np.arange(L))
    got = [np.zeros_like(a) for a in whole]
    covered = np.zeros(L, dtype=np.int64)
    costs = []
    for g in range(G):
        (b0, e0), (b1, e1) = dsa.zigzag_ranges(L, G, g)
        rows = np.concatenate([np.arange(b0, e0), np.arange(b1, e1)])
        assert np.array_equal(rows, oracle.zigzag_shard(L, G, g))
        res = run_rows(dsa, inp, d, rows)
        for a, r in zip(got, res):
            a[rows] = r
        covered[rows] += 1
        costs.append(oracle.causal_cost(rows, P))
    log(f"  chunk L={L} P={P} G={G}: shard causal costs {costs}")
    assert np.all(covered == 1)
    assert np.array_equal(got[0], whole[0])
    assert np.array_equal(got[1].view(np.uint32), whole[1].view(np.uint32))
    Og = oracle.decode(got[2].view(np.uint16), "bf16")
    Ow = oracle.decode(whole[2].view(np.uint16), "bf16")
    assert np.max(np.abs(Og - Ow)) <= TOL_O
    assert np.max(np.abs(got[3].astype(np.float64) - whole[3])) <= TOL_LSE
    sample = sorted({0, L // 3, L - 1, int(oracle.zigzag_shard(L, G, G - 1)[0])})
    refs = oracle.indexer_topk(inp, sample)
    res = oracle.check_topk(got[0], refs)
    assert res.ok, res.msgs[:5]
    Oref, Lref = oracle.sfa(inp, got[0], sample)
    O = oracle.decode(got[2][sample].view(np.uint16), "bf16")
    c = oracle.check_attention(O, Oref, TOL_O, got[3][sample].astype(np.float64), Lref, TOL_LSE)
    assert c.ok, c.msgs
