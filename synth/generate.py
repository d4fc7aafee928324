"""Seeded generation of the stored tensors for one workload.

Everything is drawn from numpy's PCG64 with a fixed seed and a fixed chunking, so the same
(spec, seed) always yields the same bits.  Values are drawn in float32 and stored as:

* fp32: as drawn;
* bf16: rounded to nearest-even by torch's CPU conversion, kept as raw uint16 bits;
* fp8-e4m3 (OCP "fn" variant, max 448) with one fp32 scale per token: the scale is the
  row's largest magnitude divided by 448 (an all-zero row gets scale 1), and the codes are
  torch's CPU conversion of value/scale, kept as raw uint8 bits.

Pools are laid out physically: row = physical_block * block_size + slot, one block table
shared by the indexer-key pool, its scales and the latent-KV pool.  Slots past a sequence's
end and whole unused blocks hold NaN, so any read of them shows up in the results.
Unused block-table columns point at a NaN block.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from .configs import Spec

_CHUNK_ROWS = 1 << 16
F32_NAN = np.float32("nan")
BF16_NAN = np.uint16(0x7FC0)
FP8_NAN = np.uint8(0x7F)


@dataclass
class Inputs:
    spec: Spec
    q_idx: np.ndarray                 # [T, H_I, D_I]  float32 | uint16 (bf16 bits)
    w: np.ndarray                     # [T, H_I] float32
    k_pool: np.ndarray                # [rows, D_I]  float32 | uint16 | uint8 (fp8 codes)
    k_scale: Optional[np.ndarray]     # [rows] float32, fp8 keys only
    q_sfa: np.ndarray                 # [T, H, d_qk]  float32 | uint16
    kv_pool: np.ndarray               # [rows, d_qk]  float32 | uint16
    block_table: Optional[np.ndarray] # [num_seqs, max_blocks] int32, or None (contiguous)
    seq_stride: int                   # contiguous layout: rows between sequences
    q_seq: np.ndarray                 # [T] int32
    q_visible: np.ndarray             # [T] int32
    seed: int

    @property
    def block_size(self) -> int:
        return self.spec.block_size


def _f32_normal(rng, shape, std) -> np.ndarray:
    out = np.empty(shape, dtype=np.float32)
    flat = out.reshape(shape[0], -1)
    for lo in range(0, shape[0], _CHUNK_ROWS):
        hi = min(shape[0], lo + _CHUNK_ROWS)
        flat[lo:hi] = rng.standard_normal(flat[lo:hi].shape, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 raw bits (round to nearest even), via torch's CPU conversion."""
    out = np.empty(x.shape, dtype=np.uint16)
    xf = x.reshape(-1)
    of = out.reshape(-1)
    step = 1 << 24
    for lo in range(0, xf.size, step):
        t = torch.from_numpy(np.ascontiguousarray(xf[lo:lo + step]))
        of[lo:lo + step] = t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return out


def to_fp8_per_token(x: np.ndarray):
    """float32 [rows, D] -> (uint8 e4m3fn codes [rows, D], float32 scales [rows])."""
    amax = np.abs(x).max(axis=1)
    scale = (amax / np.float32(448.0)).astype(np.float32)
    scale[amax == 0] = np.float32(1.0)
    codes = np.empty(x.shape, dtype=np.uint8)
    for lo in range(0, x.shape[0], _CHUNK_ROWS):
        hi = min(x.shape[0], lo + _CHUNK_ROWS)
        y = torch.from_numpy(np.ascontiguousarray(x[lo:hi] / scale[lo:hi, None]))
        codes[lo:hi] = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return to_bf16_bits(x)
    raise ValueError(dtype)


def _nan_of(arr: np.ndarray):
    return {np.float32: F32_NAN, np.uint16: BF16_NAN, np.uint8: FP8_NAN}[arr.dtype.type]


def make_inputs(spec: Spec, seed: int, *, sfa_dist: str = "config",
                poison: bool = True, with_sfa: bool = True) -> Inputs:
    """Draw every stored tensor of `spec` from PCG64(seed).

    sfa_dist: "config" draws the SFA query and latent rows as the workload states
    (N(0, 1/576)); "sharp" draws latent rows from N(0, 0.25^2) and queries from N(0, 8^2),
    which gives logits of standard deviation about 2, so that the softmax is far from
    uniform and wrong attention outputs are far from right ones.
    """
    rng = np.random.default_rng(np.random.PCG64(seed))
    T = spec.num_queries
    B = spec.num_seqs
    lens = np.asarray(spec.seq_lens, dtype=np.int64)
    q_seq = np.asarray(spec.q_seq, dtype=np.int32)
    q_vis = np.asarray(spec.q_visible, dtype=np.int32)
    if np.any(q_vis < 1) or np.any(q_vis > lens[q_seq]):
        raise ValueError("every query must see between 1 and its sequence's length")

    # ---- layout -----------------------------------------------------------------------
    bs = spec.block_size
    if bs > 0:
        nblk = -(-lens // bs)
        extra = max(1, spec.extra_blocks)
        total_blocks = int(nblk.sum()) + extra
        perm = rng.permutation(total_blocks) if spec.permute else np.arange(total_blocks)
        max_blocks = int(nblk.max()) + 1
        poison_block = int(perm[-1])          # one of the unused blocks
        bt = np.full((B, max_blocks), poison_block, dtype=np.int32)
        off = 0
        for b in range(B):
            bt[b, :nblk[b]] = perm[off:off + nblk[b]]
            off += int(nblk[b])
        unused_blocks = perm[off:]
        rows = total_blocks * bs
        stride = 0
    else:
        bt = None
        stride = int(lens.max())
        rows = B * stride

    def poison_rows(arr):
        if not poison:
            return
        nan = _nan_of(arr)
        if bs > 0:
            for blk in unused_blocks:
                arr[int(blk) * bs:(int(blk) + 1) * bs] = nan
            for b in range(B):
                tail = int(lens[b] % bs)
                if tail:
                    blk = int(bt[b, nblk[b] - 1])
                    arr[blk * bs + tail:(blk + 1) * bs] = nan
        else:
            for b in range(B):
                arr[b * stride + int(lens[b]):(b + 1) * stride] = nan

    # ---- indexer query, head weights, keys ---------------------------------------------
    q_idx = _store(_f32_normal(rng, (T, spec.idx_heads, spec.idx_dim), spec.q_std), spec.q_dtype)
    w = _f32_normal(rng, (T, spec.idx_heads), spec.w_std)
    kf = _f32_normal(rng, (rows, spec.idx_dim), spec.k_std)
    if spec.k_dtype == "fp8":
        k_pool, k_scale = to_fp8_per_token(kf)
        poison_rows(k_scale)
    else:
        k_pool, k_scale = _store(kf, spec.k_dtype), None
    del kf
    poison_rows(k_pool)

    # ---- SFA query and latent KV --------------------------------------------------------
    if sfa_dist == "config":
        sq, skv = spec.sfa_q_std, spec.sfa_kv_std
    elif sfa_dist == "sharp":
        sq, skv = 8.0, 0.25
    else:
        raise ValueError(sfa_dist)
    if with_sfa:
        q_sfa = _store(_f32_normal(rng, (T, spec.sfa_heads, spec.d_qk), sq), spec.kv_dtype)
        kv_pool = _store(_f32_normal(rng, (rows, spec.d_qk), skv), spec.kv_dtype)
        poison_rows(kv_pool)
    else:
        q_sfa = kv_pool = None

    return Inputs(spec=spec, q_idx=q_idx, w=w, k_pool=k_pool, k_scale=k_scale,
                  q_sfa=q_sfa, kv_pool=kv_pool, block_table=bt, seq_stride=stride,
                  q_seq=q_seq, q_visible=q_vis, seed=seed)


@dataclass
class PrologInputs:
    """Hidden vectors and weights of the indexer prolog (bf16 bits) and the key's gain."""
    x: np.ndarray        # [T, d_x] uint16
    w_proj: np.ndarray   # [d_x, H*D + D + H] uint16
    gain: np.ndarray     # [D] float32
    n_heads: int
    head_dim: int
    eps: float


def make_prolog_inputs(n_tokens: int, d_x: int, n_heads: int, head_dim: int, seed: int,
                       eps: float = 1e-6) -> PrologInputs:
    """x ~ N(0, 1) and W ~ N(0, 1/d_x), so every projection is about N(0, 1); gain ~
    U(0.5, 1.5)."""
    rng = np.random.default_rng(np.random.PCG64(seed))
    N = n_heads * head_dim + head_dim + n_heads
    x = to_bf16_bits(_f32_normal(rng, (n_tokens, d_x), 1.0))
    w = to_bf16_bits(_f32_normal(rng, (d_x, N), 1.0 / math.sqrt(d_x)))
    gain = rng.uniform(0.5, 1.5, head_dim).astype(np.float32)
    return PrologInputs(x, w, gain, n_heads, head_dim, eps)
