"""Logical (sequence, position) -> physical pool row, written out plainly.

TEST INFRASTRUCTURE (see the package header).

The indexer reads the paged key cache and SFA the paged KV cache ("Day0 Adaptation and
Performance Optimization for Novel Long-Sequence Reasoning Models", section 3; "Large Model
Inference Acceleration: Day-0 Adaptation...", section 1.1).  One block table serves every
pool: position s of sequence b lives in physical block block_table[b, s // block_size], slot
s % block_size, i.e. row block * block_size + slot.  Without a block table the sequences are
contiguous: row b * seq_stride + s.
"""
from __future__ import annotations

import numpy as np


def logical_rows(block_table, block_size: int, seq_stride: int, b: int, positions) -> np.ndarray:
    pos = np.asarray(positions, dtype=np.int64)
    if block_table is None or block_size == 0:
        return b * int(seq_stride) + pos
    blocks = block_table[b].astype(np.int64)[pos // block_size]
    return blocks * block_size + pos % block_size


def depage(pool: np.ndarray, block_table, block_size: int, seq_stride: int, b: int, n: int) -> np.ndarray:
    """Rows 0..n-1 of sequence b, in logical order (a copy)."""
    return pool[logical_rows(block_table, block_size, seq_stride, b, np.arange(n))]
