"""Workload shapes for the DSA sparse-attention hot path.

Each workload fixes: how many sequences there are and how long each is, which sequence
each query belongs to and how many cached positions it may see (its visible prefix,
counting its own position), the lightning-indexer geometry (heads x dims, Top-K), the
storage formats of queries and keys, the MLA latent geometry of Sparse Flash Attention
(576-wide q/k rows whose first 512 columns are the value), and the paged layout (64-token
blocks scattered by a random block-table permutation).

Sources: "Day0 Adaptation and Performance Optimization for Novel Long-Sequence Reasoning
Models", section 1 (indexer + Top-K + SFA on top of MLA) and section 3 (the indexer reads the
paged K cache, SFA reads the main KV at the selected positions); "Large Model Inference
Acceleration: Day-0 Adaptation...", section 1.1 (fused operator reads the paged cache
directly).  The sizes themselves are the five benchmark workloads of this project.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np


@dataclass(frozen=True)
class Spec:
    name: str
    seq_lens: tuple            # tokens stored per sequence
    q_seq: tuple               # sequence id of every query
    q_visible: tuple           # visible prefix length V_t of every query (>= 1)
    idx_heads: int = 64        # H_I
    idx_dim: int = 128         # D_I
    top_k: int = 2048          # K
    q_dtype: str = "bf16"      # indexer query storage: f32 | bf16
    k_dtype: str = "bf16"      # indexer key storage: f32 | bf16 | fp8 (per-token fp32 scale)
    sfa_heads: int = 128       # H
    d_qk: int = 576            # latent q/k width (512 nope + 64 rope)
    d_v: int = 512             # value width = first d_v columns of the latent row
    kv_dtype: str = "bf16"     # SFA query / latent KV / output storage: f32 | bf16
    block_size: int = 64       # tokens per page; 0 = contiguous per-sequence layout
    permute: bool = True       # scatter physical blocks by a random permutation
    extra_blocks: int = 2      # unused, NaN-poisoned blocks appended to the pools
    q_std: float = 1.0 / math.sqrt(128)
    k_std: float = 1.0 / math.sqrt(128)
    w_std: float = 1.0 / math.sqrt(64)
    sfa_q_std: float = 1.0 / math.sqrt(576)
    sfa_kv_std: float = 1.0 / math.sqrt(576)
    softmax_scale: float = 1.0 / math.sqrt(576)

    @property
    def num_queries(self) -> int:
        return len(self.q_seq)

    @property
    def num_seqs(self) -> int:
        return len(self.seq_lens)

    @property
    def max_visible(self) -> int:
        return int(max(self.q_visible))

    def k_eff(self, t: int) -> int:
        return min(self.top_k, int(self.q_visible[t]))


def _decode_spec(name, lens, **kw) -> Spec:
    lens = tuple(int(x) for x in lens)
    return Spec(name=name, seq_lens=lens, q_seq=tuple(range(len(lens))), q_visible=lens, **kw)


def tiny_decode_fp32() -> Spec:
    """Batch 1, context 4096, fp32 throughout; indexer 8 x 64, head weights N(0, 1/8);
    q, k ~ N(0, 1/d); Top-K 256; SFA 16 heads, 576/512, scale 1/sqrt(576); contiguous KV."""
    return _decode_spec(
        "tiny_decode_fp32", [4096], idx_heads=8, idx_dim=64, top_k=256,
        q_dtype="f32", k_dtype="f32", sfa_heads=16, kv_dtype="f32",
        block_size=0, permute=False, extra_blocks=0,
        q_std=1 / 8.0, k_std=1 / 8.0, w_std=1 / math.sqrt(8))


def decode_bf16_32k() -> Spec:
    """Decode batch 32 x 32768 context, bf16; indexer 64 x 128, Top-K 2048; SFA 128 heads;
    64-token pages in a random block-table permutation."""
    return _decode_spec("decode_bf16_32k", [32768] * 32)


def prefill_chunk_bf16() -> Spec:
    """Chunked prefill: one sequence, 4096 new query tokens appended to a 65536-token
    causal context; query i sees positions [0, 65536 + i + 1)."""
    prefix, new = 65536, 4096
    total = prefix + new
    return Spec(name="prefill_chunk_bf16", seq_lens=(total,), q_seq=(0,) * new,
                q_visible=tuple(prefix + i + 1 for i in range(new)))


def decode_fp8_128k(seed: int = 4) -> Spec:
    """Quantized decode: batch 8, per-sequence context uniform in [64K, 128K]; indexer keys
    fp8-e4m3 with one fp32 scale per token (values N(0,1) before quantization); bf16
    queries; Top-K 2048; SFA bf16 128 heads, 576/512 latent."""
    rng = np.random.default_rng(np.random.PCG64(seed * 1000003 + 17))
    lens = rng.integers(65536, 131072, size=8, endpoint=True)
    return _decode_spec("decode_fp8_128k", lens, k_dtype="fp8", k_std=1.0)


def decode_fp8_1m() -> Spec:
    """Million-token decode: batch 1, context 1048576, fp8-e4m3 indexer keys with per-token
    scales, Top-K 2048; SFA bf16 128 heads over a ~1.2 GB paged latent cache."""
    return _decode_spec("decode_fp8_1m", [1 << 20], k_dtype="fp8", k_std=1.0)


def prefill_causal_16k() -> Spec:
    """Causal prefill with no prefix: one sequence of 16384 new tokens, query i sees
    positions [0, i + 1), so the first 2047 queries see fewer than K positions and later
    queries cost more (the load the zigzag layout balances); bf16, Top-K 2048."""
    n = 16384
    return Spec(name="prefill_causal_16k", seq_lens=(n,), q_seq=(0,) * n,
                q_visible=tuple(range(1, n + 1)))


WORKLOADS = {
    1: tiny_decode_fp32,
    2: decode_bf16_32k,
    3: prefill_chunk_bf16,
    4: decode_fp8_128k,
    5: decode_fp8_1m,
    6: prefill_causal_16k,
}


def workload(n: int) -> Spec:
    return WORKLOADS[n]()


def scaled_spec(base: Spec, *, seq_lens=None, q_seq=None, q_visible=None, name=None, **kw) -> Spec:
    """A copy of `base` with other lengths (decode: one query per sequence seeing all of it,
    unless q_seq/q_visible are given) or other fields."""
    if seq_lens is not None:
        seq_lens = tuple(int(x) for x in seq_lens)
        if q_seq is None:
            q_seq = tuple(range(len(seq_lens)))
        if q_visible is None:
            q_visible = tuple(seq_lens[s] for s in q_seq)
    upd = dict(kw)
    if seq_lens is not None:
        upd["seq_lens"] = seq_lens
    if q_seq is not None:
        upd["q_seq"] = tuple(int(x) for x in q_seq)
    if q_visible is not None:
        upd["q_visible"] = tuple(int(x) for x in q_visible)
    upd["name"] = name or (base.name + "_scaled")
    return dataclasses.replace(base, **upd)
