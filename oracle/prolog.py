"""The indexer prolog by its definition: the projections that make the indexer's query, key
and head weights from a token's hidden vector, and the key's normalization.

TEST INFRASTRUCTURE (see the package header).

The pages list the steps and run them on parallel streams: query projection, key
normalization (RMSNorm), query quantization and head-weight projection ("Day0 Adaptation
and Performance Optimization for Novel Long-Sequence Reasoning Models", section 3; "Large
Model Inference Acceleration: Day-0 Adaptation...", section 1.2; "Optimizing and Deploying
Ultra-Long Sequence Inference Architectures", section I).  Readings where they are silent:
all three projections read the same hidden vector x (bf16, width d_x) through one bf16
weight matrix W of d_x rows whose columns are the query (head-major, H * D), the key (D)
and the head weights (H); the key is RMS-normalized with a learned fp32 gain:

    Y = x W                     (float64 here)
    q = Y[:, :H D]              reshaped [T, H, D]
    k = Y[:, H D : H D + D] / sqrt(mean(Y[:, H D : H D + D]^2) + eps) * gain
    w = Y[:, H D + D :]

The query's quantization is that of the index keys: none for bf16 or per-token fp8 keys
(the query stays bf16), the MXFP8 group-32 quantization for MXFP8 keys; the key is then
stored by the cache writer's format (see codecs).
"""
from __future__ import annotations

import numpy as np

from .codecs import decode_bf16


def project(x_bits: np.ndarray, w_bits: np.ndarray) -> np.ndarray:
    """bf16 bits x [T, d_x] and W [d_x, N] -> Y = x W in float64."""
    return decode_bf16(x_bits) @ decode_bf16(w_bits)


def rms_norm(v: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """Each row divided by the root of (its mean square + eps), times gain; float64."""
    v = np.asarray(v, dtype=np.float64)
    r = np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps)
    return v / r * np.asarray(gain, dtype=np.float64)


def indexer_prolog(x_bits, w_bits, gain, eps: float, n_heads: int, head_dim: int):
    """-> (q [T, H, D], k [T, D], w [T, H]) float64."""
    Y = project(x_bits, w_bits)
    HD = n_heads * head_dim
    T = Y.shape[0]
    q = Y[:, :HD].reshape(T, n_heads, head_dim)
    k = rms_norm(Y[:, HD:HD + head_dim], gain, eps)
    w = Y[:, HD + head_dim:HD + head_dim + n_heads]
    return q, k, w
