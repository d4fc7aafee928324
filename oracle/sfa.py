"""Sparse Flash Attention by its plain definition: dense softmax over the selected rows.

TEST INFRASTRUCTURE (see the package header).

SFA reads the main-attention KV cache only at the positions the indexer selected and runs
attention over them ("Day0 Adaptation and Performance Optimization for Novel Long-Sequence
Reasoning Models", section 1 and 3; "Day0 Adaptation and Sparse Attention Optimization for
Long-Sequence LLM Inference", section 4).  The cache is the MLA latent cache: one d_qk-wide
row per token (512 "nope" + 64 "rope" columns) serves as the key, and its first d_v = 512
columns serve as the value.  For query t with SFA query q[t] (H x d_qk) and selected rows R
(n x d_qk; entries equal to -1 in the index list are skipped, repeated entries count once
per occurrence):

    Z = scale * q[t] @ R^T          (H x n)
    P = exp(Z - max_j Z)            per head
    O = (P @ R[:, :d_v]) / sum_j P  (H x d_v)
    LSE = max_j Z + log(sum_j P)    natural log

With no row at all, O = 0 and LSE = -inf.  Float64 throughout.  With fp8 latent rows
(kv_dtype "fp8": bf16 queries, rows quantized per 128-column tile, see codecs) R is the
dequantized row, code times tile scale, exactly.
"""
from __future__ import annotations

import numpy as np

from .codecs import decode
from .paging import logical_rows


def sfa_dense(q: np.ndarray, rows: np.ndarray, scale: float, d_v: int):
    """q [H, d_qk], rows [n, d_qk] float64 -> (O [H, d_v], lse [H]) float64."""
    H = q.shape[0]
    if rows.shape[0] == 0:
        return np.zeros((H, d_v)), np.full(H, -np.inf)
    Z = scale * (q @ rows.T)
    m = Z.max(axis=1, keepdims=True)
    P = np.exp(Z - m)
    l = P.sum(axis=1)
    O = (P @ rows[:, :d_v]) / l[:, None]
    lse = m[:, 0] + np.log(l)
    return O, lse


def sfa_query(inp, t: int, idx_row: np.ndarray):
    """Attention of query t over the logical positions in idx_row (-1 skipped)."""
    spec = inp.spec
    b = int(inp.q_seq[t])
    pos = np.asarray(idx_row, dtype=np.int64)
    pos = pos[pos != -1]
    rows = logical_rows(inp.block_table, inp.block_size, inp.seq_stride, b, pos)
    fp8 = spec.kv_dtype == "fp8"
    R = decode(inp.kv_pool[rows], "fp8_rows" if fp8 else spec.kv_dtype)
    q = decode(inp.q_sfa[t], "bf16" if fp8 else spec.kv_dtype)
    return sfa_dense(q, R, spec.softmax_scale, spec.d_v)


def sfa(inp, idx: np.ndarray, queries=None):
    """idx [T, K] -> (O [len(queries), H, d_v], lse [len(queries), H])."""
    if queries is None:
        queries = range(inp.spec.num_queries)
    outs, lses = [], []
    for t in queries:
        o, l = sfa_query(inp, int(t), idx[int(t)])
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)
