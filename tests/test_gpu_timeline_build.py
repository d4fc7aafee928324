"""The phase-stamp measurement build (libdsa_timeline.so) computes what libdsa.so computes.

The timeline profiles are taken with a second build of the same sources, whose kernels also
write a clock reading per phase and workgroup.  One decode step (indexer then sparse attention,
the 64-head decode kernel and its combine) is run through both libraries on the same inputs:
the index lists and the attention outputs must be bit-identical, and the stamp buffer must hold
a start stamp for every indexer and attention workgroup of the step.  Skipped when the
measurement build has not been made (python -m sparse_indexed_attention_amd.build --timeline)."""
import os

import numpy as np
import pytest

from synth import make_inputs, scaled_spec, workload
from synth.device import to_device
from tests.gpu_util import layout_of

pytestmark = pytest.mark.gpu

TL_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                       "sparse_indexed_attention_amd", "libdsa_timeline.so")


def test_timeline_build_matches_the_library(dsa):
    import torch
    if not os.path.exists(TL_PATH):
        pytest.skip("libdsa_timeline.so not built")
    spec = scaled_spec(workload(4), seq_lens=[40000, 9000, 70000, 3000])
    inp = make_inputs(spec, seed=41)
    d = to_device(inp)
    T, K = spec.num_queries, spec.top_k
    V = np.asarray(inp.q_visible)

    def step():
        wsi = dsa.zeroed_workspace(dsa.indexer_workspace_bytes(T, d.max_visible, K), "cuda")
        wss = dsa.zeroed_workspace(dsa.sfa_workspace_bytes(T, spec.sfa_heads, K, spec.d_v), "cuda")
        lay = layout_of(dsa, d)
        idx, _ = dsa.indexer_topk(d.q_idx, d.w, d.k_pool, d.k_scale, lay, d.q_seq, d.q_visible,
                                  d.max_visible, K, want_score=False, workspace=wsi,
                                  total_visible=int(V.sum()))
        out, lse = dsa.sparse_attn(d.q_sfa, d.kv_pool, idx, lay, d.q_seq, spec.softmax_scale,
                                   spec.d_v, workspace=wss)
        torch.cuda.synchronize()
        return idx.clone(), out.clone(), lse.clone()

    want = step()
    saved = dsa._lib
    try:
        dsa._lib = None
        dsa.load(TL_PATH)
        buf = torch.zeros(dsa.timeline_bytes() // 8, dtype=torch.int64, device="cuda")
        dsa.timeline_register(buf)
        got = step()
        dsa.timeline_register(None)
    finally:
        dsa._lib = saved
    for a, b, name in zip(want, got, ("index lists", "attention output", "LSE")):
        assert torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8)), name
    stamps = buf.view(3, 4096, -1).cpu().numpy()
    started = (stamps[:, :, 0] > 0).sum(axis=1)
    assert started[0] >= T          # every indexer workgroup of the compact launch (one per split)
    assert started[1] >= T * 2      # at least one slice per (query, 64-head group)
    assert started[2] > 0           # the combine kernel ran
