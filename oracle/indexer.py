"""Lightning-indexer scores and exact Top-K, by the plain definition.

TEST INFRASTRUCTURE (see the package header).

What is computed (for one query t of sequence b that sees positions [0, V)):

    x[h, s] = q[t, h, :] . k[b, s, :]                  per-head dot product
    S[s]    = sum_h  w[t, h] * max(x[h, s], 0)          ReLU, then head-weighted sum
    S32[s]  = S[s] rounded to fp32 (nearest even), -0 taken as +0
    Top-K   = the K_eff = min(K, V) positions with the largest S32, the lower position
              first among equal scores

The three steps follow the pages' description of the indexer as relevance scores, combined
under per-head weights, then a Top-K selection ("Day0 Adaptation and Performance Optimization for Novel Long-Sequence Reasoning
Models", section 3; "Optimizing and Deploying Ultra-Long Sequence Inference Architectures",
section I; "Large Model Inference Acceleration: Day-0 Adaptation...", section 1.1, where the
per-head scores are the Batch x Head x Seq intermediate of section 2.1).  The pages give no
formula; the per-head dot product, ReLU, the head weights and the lowest-position tie-break
are this project's reading.  One key vector per token is shared by all indexer heads.  fp8
keys are dequantized (code value times the token's fp32 scale) before the dot product.
MXFP8 keys (k_dtype "mxfp8": codes and one E8M0 byte per 32 dims, see codecs) are
dequantized the same way, and the query is then quantized to MXFP8 too, per head and group
of 32 dims, before the dot product: the pages quantize both index Q and K dynamically.
Everything is float64; products of bf16/fp8/fp32 operands are exact in float64.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np

from .codecs import decode, decode_mxfp8, quantize_mxfp8
from .paging import logical_rows

_POS_CHUNK = 1 << 16     # positions are scored independently; the loop only bounds memory


def index_scores(q: np.ndarray, w: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """q [H_I, D_I], w [H_I], keys [V, D_I] (all float64) -> S [V] float64."""
    V = keys.shape[0]
    S = np.empty(V, dtype=np.float64)
    for lo in range(0, V, _POS_CHUNK):
        x = keys[lo:lo + _POS_CHUNK] @ q.T            # [n, H_I]: x[s, h] = q_h . k_s
        S[lo:lo + _POS_CHUNK] = np.maximum(x, 0.0) @ w
    return S


def to_fp32_score(S: np.ndarray) -> np.ndarray:
    S32 = S.astype(np.float32)
    S32[S32 == 0] = np.float32(0.0)
    return S32


def topk_order(S32: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest S32, score descending then position ascending (full sort)."""
    V = S32.shape[0]
    order = np.lexsort((np.arange(V), -S32.astype(np.float64)))
    return order[:k]


@dataclass
class IndexerResult:
    t: int
    k_eff: int
    idx: np.ndarray          # [K] int64: selected positions in rank order, then -1
    S32: np.ndarray          # [V] float32 scores of every visible position
    kth: np.float32          # score of the K_eff-th selected position
    band: np.ndarray         # [V] bool: |S32 - kth| <= 1e-6 * |kth|


def query_keys(inp, t: int) -> np.ndarray:
    """Dequantized float64 keys [V_t, D_I] of query t, in logical order."""
    b = int(inp.q_seq[t])
    V = int(inp.q_visible[t])
    rows = logical_rows(inp.block_table, inp.block_size, inp.seq_stride, b, np.arange(V))
    if inp.spec.k_dtype == "mxfp8":
        return decode_mxfp8(inp.k_pool[rows], inp.k_scale[rows])
    keys = decode(inp.k_pool[rows], inp.spec.k_dtype)
    if inp.spec.k_dtype == "fp8":
        keys = keys * inp.k_scale[rows].astype(np.float64)[:, None]
    return keys


def indexer_topk_query(inp, t: int, S: Optional[np.ndarray] = None) -> IndexerResult:
    spec = inp.spec
    V = int(inp.q_visible[t])
    if S is None:
        q = decode(inp.q_idx[t], spec.q_dtype)
        if spec.k_dtype == "mxfp8":
            q = decode_mxfp8(*quantize_mxfp8(q.astype(np.float32)))
        w = inp.w[t].astype(np.float64)
        S = index_scores(q, w, query_keys(inp, t))
    S32 = to_fp32_score(S)
    k_eff = min(spec.top_k, V)
    sel = topk_order(S32, k_eff)
    idx = np.full(spec.top_k, -1, dtype=np.int64)
    idx[:k_eff] = sel
    kth = S32[sel[-1]]
    band = np.abs(S32.astype(np.float64) - float(kth)) <= 1e-6 * abs(float(kth))
    return IndexerResult(t=t, k_eff=k_eff, idx=idx, S32=S32, kth=kth, band=band)


def indexer_topk(inp, queries: Optional[Sequence[int]] = None) -> List[IndexerResult]:
    if queries is None:
        queries = range(inp.spec.num_queries)
    return [indexer_topk_query(inp, int(t)) for t in queries]
