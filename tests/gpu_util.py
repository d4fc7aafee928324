"""GPU-test helpers: run the HIP path through the C-ABI binding on generated inputs."""
from __future__ import annotations

import math

import numpy as np

import oracle
from synth.device import bits_of, to_device


def layout_of(m, d):
    if d.block_table is not None:
        return m.make_layout(d.block_table, d.block_size, pool_rows=d.pool_rows)
    return m.make_layout(None, 0, seq_stride=d.seq_stride, num_seqs=d.spec.num_seqs,
                         pool_rows=d.pool_rows)


def run_indexer(m, inp, d=None, *, top_k=None, workspace=None, total_visible="exact"):
    """-> (idx int64 [T, K], score float32 [T, K]) as numpy.  total_visible: the launch hint,
    by default the true sum of the visible lengths (as the benchmark passes it)."""
    import torch
    d = d or to_device(inp)
    K = top_k or inp.spec.top_k
    tv = int(np.sum(inp.q_visible, dtype=np.int64)) if total_visible == "exact" else int(total_visible)
    idx, score = m.indexer_topk(d.q_idx, d.w, d.k_pool, d.k_scale, layout_of(m, d), d.q_seq,
                                d.q_visible, d.max_visible, K, workspace=workspace,
                                total_visible=tv)
    torch.cuda.synchronize()
    return idx.cpu().numpy().astype(np.int64), score.cpu().numpy()


def run_sfa(m, inp, idx, d=None, *, workspace=None):
    """idx: numpy [T, K] -> (O float64 [T, H, d_v], lse float64 [T, H])."""
    import torch
    d = d or to_device(inp)
    ti = torch.from_numpy(np.ascontiguousarray(idx.astype(np.int32))).to(d.q_sfa.device)
    out, lse = m.sparse_attn(d.q_sfa, d.kv_pool, ti, layout_of(m, d), d.q_seq,
                             inp.spec.softmax_scale, inp.spec.d_v, workspace=workspace)
    torch.cuda.synchronize()
    O = oracle.decode(bits_of(out), "bf16" if inp.spec.kv_dtype == "fp8" else inp.spec.kv_dtype)
    return O, lse.cpu().numpy().astype(np.float64)


def score_error(score_row, idx_row, ref):
    """Largest |GPU score - oracle fp32 score| over the selected positions, relative to the
    scale of the scores: the larger of |K-th score| (the scale of the 1e-6 tie band) and the
    RMS score of the query (|K-th| alone goes to 0 when K_eff is a large share of V)."""
    k = ref.k_eff
    pos = idx_row[:k]
    d = np.abs(score_row[:k].astype(np.float64) - ref.S32[pos].astype(np.float64))
    rms = float(np.sqrt(np.mean(ref.S32.astype(np.float64) ** 2)))
    return float(d.max() / max(abs(float(ref.kth)), rms, 1e-30)) if k else 0.0


def log(msg):
    print(msg, flush=True)
