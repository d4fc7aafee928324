"""CPU oracle for the DSA indexer -> Top-K -> Sparse Flash Attention path.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU-baseline leg
may import this package.  The product path (the HIP library and its Python binding) never
calls it and shares no code with it.

It computes the plain definition of what the path computes, in float64 NumPy, with no
blocking, fusion or reordering:

* the lightning indexer scores every visible cached position against the query with
  per-head dot products, applies ReLU per head and sums the heads under the query's head
  weights ("Day0 Adaptation and Performance Optimization for Novel Long-Sequence Reasoning
  Models", section 3; "Optimizing and Deploying Ultra-Long Sequence Inference
  Architectures", section I; "Large Model Inference Acceleration: Day-0 Adaptation...",
  section 1.1);
* Top-K keeps the K highest fp32 scores, lowest position first among equal scores, by a
  full sort;
* Sparse Flash Attention is dense softmax attention restricted to the selected rows of the
  MLA latent cache, the value being the first d_v columns of each row ("Day0 Adaptation and
  Sparse Attention Optimization for Long-Sequence LLM Inference", section 4);
* the zigzag head-tail sharding of a causal chunk (see zigzag.py);
* the indexer prolog: projections of the hidden vector and the key's RMSNorm (prolog.py).

Every function is pinned by the CPU tests against something other than itself (closed
forms, brute force, library routines); see tests/test_oracle_*.py.
"""
from .codecs import (decode, decode_bf16, decode_fp8_e4m3, fp8_e4m3_table, encode_bf16_rne,
                     encode_fp8_e4m3, quantize_fp8_per_token, kv_fp8_tile_scale,
                     quantize_kv_fp8_rows, decode_kv_fp8_rows, KV_FP8_ROW_BYTES,
                     mx_scale_bytes, quantize_mxfp8, decode_mxfp8)
from .paging import logical_rows, depage
from .indexer import (index_scores, to_fp32_score, topk_order, IndexerResult,
                      indexer_topk_query, indexer_topk)
from .sfa import sfa_dense, sfa_query, sfa
from .compare import TopkCheck, check_topk_row, check_topk, AttnCheck, check_attention
from .zigzag import zigzag_segments, zigzag_shard, contiguous_shard, causal_cost
from .prolog import project, rms_norm, indexer_prolog

__all__ = [
    "decode", "decode_bf16", "decode_fp8_e4m3", "fp8_e4m3_table", "encode_bf16_rne",
    "encode_fp8_e4m3", "quantize_fp8_per_token", "kv_fp8_tile_scale", "quantize_kv_fp8_rows",
    "decode_kv_fp8_rows", "KV_FP8_ROW_BYTES", "mx_scale_bytes", "quantize_mxfp8",
    "decode_mxfp8", "logical_rows", "depage", "index_scores",
    "to_fp32_score", "topk_order", "IndexerResult", "indexer_topk_query", "indexer_topk",
    "sfa_dense", "sfa_query", "sfa", "TopkCheck", "check_topk_row", "check_topk",
    "AttnCheck", "check_attention", "zigzag_segments", "zigzag_shard", "contiguous_shard",
    "causal_cost", "project", "rms_norm", "indexer_prolog",
]
