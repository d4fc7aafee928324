"""The hot path under HIP graph capture: one decode step (dsa_indexer_topk then
dsa_sparse_attn) captured once and replayed several times, with eager steps on other inputs
in between, must give bit-identical outputs to the eager step every time.  The library
records no memset and allocates nothing in these calls; the indexer's arrival counters
reset themselves, so a replay finds its workspace as the previous one left it."""
import numpy as np
import pytest

from synth import make_inputs, scaled_spec, workload
from synth.device import to_device
from tests.gpu_util import layout_of, log

pytestmark = pytest.mark.gpu


def test_captured_step_replays_match_eager(dsa):
    import torch
    spec = scaled_spec(workload(4), seq_lens=[30000, 12000, 70000, 2500])
    inp = make_inputs(spec, seed=31)
    other = make_inputs(spec, seed=32)
    d, d2 = to_device(inp), to_device(other)
    T, K = spec.num_queries, spec.top_k
    V = np.asarray(inp.q_visible)
    wsi = dsa.zeroed_workspace(dsa.indexer_workspace_bytes(T, d.max_visible, K), "cuda")
    wss = dsa.zeroed_workspace(dsa.sfa_workspace_bytes(T, spec.sfa_heads, K, spec.d_v), "cuda")
    idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
    out = torch.empty((T, spec.sfa_heads, spec.d_v), dtype=d.q_sfa.dtype, device="cuda")

    def step(dd):
        lay = layout_of(dsa, dd)
        dsa.indexer_topk(dd.q_idx, dd.w, dd.k_pool, dd.k_scale, lay, dd.q_seq, dd.q_visible,
                         dd.max_visible, K, out_idx=idx, want_score=False, workspace=wsi,
                         total_visible=int(V.sum()))
        dsa.sparse_attn(dd.q_sfa, dd.kv_pool, idx, lay, dd.q_seq, spec.softmax_scale, spec.d_v,
                        out=out, want_lse=False, workspace=wss)

    step(d)
    torch.cuda.synchronize()
    want_idx, want_out = idx.clone(), out.clone()
    step(d2)
    torch.cuda.synchronize()
    other_idx = idx.clone()
    assert not torch.equal(other_idx, want_idx)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(d)                                   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(d)
    torch.cuda.synchronize()
    for r in range(4):
        idx.fill_(-7)
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, want_idx), f"replay {r}: indices differ"
        assert torch.equal(out.view(torch.int16), want_out.view(torch.int16)), f"replay {r}: output differs"
        step(d2)                                  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(idx, other_idx)
    log(f"  {T} queries: 4 replays match the eager step")
