"""Zigzag head-tail sharding of a causal chunk, by its definition.

TEST INFRASTRUCTURE (see the package header).

With causal attention a token's indexer work grows with its visible history, so cutting a
chunk of new tokens into G contiguous shards loads the last shard most.  The zigzag layout
cuts the chunk into 2G segments and gives shard g the g-th segment from the head and the
g-th from the tail, pairing short and long histories ("Day0 Adaptation and Performance
Optimization for Novel Long-Sequence Reasoning Models", section 5, whose two-device example
is [0, L/4) + [3L/4, L) and [L/4, L/2) + [L/2, 3L/4); "Large Model Inference Acceleration:
Day-0 Adaptation...", section 3.1: with N segments device 0 takes segments 1 and N, device 1
takes 2 and N-1, and so on; "Optimizing and Deploying Ultra-Long Sequence Inference
Architectures", section 3.2).  The outputs are put back in token order afterwards.

Reading where the pages are silent: the segments are as equal as possible, segment s being
[floor(s L / 2G), floor((s + 1) L / 2G)); a shard lists its head segment first.
"""
from __future__ import annotations

import numpy as np


def zigzag_segments(n_tokens: int, n_shards: int) -> list:
    """The 2G segment bounds [(begin, end)] of a chunk of n_tokens tokens."""
    m = 2 * n_shards
    return [(s * n_tokens // m, (s + 1) * n_tokens // m) for s in range(m)]


def zigzag_shard(n_tokens: int, n_shards: int, shard: int) -> np.ndarray:
    """Token indices (within the chunk) of shard `shard`: segment shard, then segment
    2G - 1 - shard."""
    seg = zigzag_segments(n_tokens, n_shards)
    head, tail = seg[shard], seg[2 * n_shards - 1 - shard]
    return np.concatenate([np.arange(*head), np.arange(*tail)]).astype(np.int64)


def contiguous_shard(n_tokens: int, n_shards: int, shard: int) -> np.ndarray:
    """The plain split the zigzag layout replaces: shard g takes [g L / G, (g + 1) L / G)."""
    return np.arange(shard * n_tokens // n_shards, (shard + 1) * n_tokens // n_shards,
                     dtype=np.int64)


def causal_cost(tokens: np.ndarray, prefix: int) -> int:
    """Positions the indexer scores for these new tokens: token i of a chunk appended to a
    prefix of P tokens sees P + i + 1 positions."""
    t = np.asarray(tokens, dtype=np.int64)
    return int(np.sum(prefix + t + 1))
