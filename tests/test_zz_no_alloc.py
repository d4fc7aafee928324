"""dsa_indexer_topk_noalloc (the indexer with the library's own device scratch array as its
workspace) against dsa_indexer_topk with a caller workspace, through the C ABI: two calls in a
row, the second on a smaller batch, must give the same index lists and scores bit for bit, and
the first also matches the oracle."""
import numpy as np
import pytest

import oracle
from synth import make_inputs, scaled_spec, workload
from synth.device import to_device
from tests.gpu_util import layout_of, log, run_indexer

pytestmark = pytest.mark.gpu


def _noalloc(dsa, inp):
    import torch
    d = to_device(inp)
    T, K = inp.spec.num_queries, inp.spec.top_k
    idx = torch.full((T, K), -7, dtype=torch.int32, device="cuda")
    score = torch.full((T, K), -7.0, dtype=torch.float32, device="cuda")
    tv = int(np.sum(inp.q_visible, dtype=np.int64))
    dsa.indexer_topk_noalloc(d.q_idx, d.w, d.k_pool, d.k_scale, layout_of(dsa, d), d.q_seq,
                             d.q_visible, d.max_visible, K, out_idx=idx, out_score=score,
                             total_visible=tv)
    torch.cuda.synchronize()
    return idx.cpu().numpy().astype(np.int64), score.cpu().numpy()


@pytest.mark.parametrize("first,second", [
    (scaled_spec(workload(4), seq_lens=[30000, 12000, 2000]),
     scaled_spec(workload(4), seq_lens=[5000, 700])),
    (scaled_spec(workload(2), seq_lens=[20000, 9000, 64, 3000]),
     scaled_spec(workload(2), seq_lens=[4100, 1], top_k=300)),
])
def test_noalloc_matches_the_workspace_entry_point(dsa, first, second):
    for n, spec in enumerate((first, second)):
        inp = make_inputs(spec, seed=40 + n, with_sfa=False)
        log(f"noalloc call {n}: T={spec.num_queries} maxV={spec.max_visible} K={spec.top_k} "
            f"keys {spec.k_dtype}")
        i1, s1 = _noalloc(dsa, inp)
        i0, s0 = run_indexer(dsa, inp)
        assert np.array_equal(i1, i0)
        assert np.array_equal(s1.view(np.uint32), s0.view(np.uint32))
        if n == 0:
            res = oracle.check_topk(i1, oracle.indexer_topk(inp))
            assert res.ok, res.msgs[:5]
