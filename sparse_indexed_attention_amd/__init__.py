"""Python binding of libdsa (the C-ABI DSA hot path for MI355X / gfx950).

Argument marshalling only: every step of the path runs in the HIP kernels of libdsa.so.
PyTorch provides device memory and the current stream.  If the library is not built, every
entry point raises; there is no fallback implementation.

Entry points mirror include/dsa.h:
    indexer_topk(...)       -> (idx [T, K] int32, score [T, K] float32 or None)
    sparse_attn(...)        -> (out [T, H, d_v], lse [T, H] float32 or None)
    store_index_keys(...), store_kv(...)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdsa.so")

DSA_F32, DSA_BF16, DSA_FP8_E4M3, DSA_MXFP8_E4M3 = 0, 1, 2, 3
DSA_MAX_TOPK = 2048
DSA_MAX_CONTEXT = 1 << 22
STATUS = {0: "DSA_OK", 1: "DSA_ERR_NULL", 2: "DSA_ERR_SHAPE", 3: "DSA_ERR_DTYPE",
          4: "DSA_ERR_UNSUPPORTED", 5: "DSA_ERR_WORKSPACE", 6: "DSA_ERR_ALIGN", 7: "DSA_ERR_HIP"}


class DsaLayout(ctypes.Structure):
    _fields_ = [("block_size", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
                ("block_table", ctypes.c_void_p), ("seq_stride", ctypes.c_int64),
                ("num_seqs", ctypes.c_int32), ("pool_rows", ctypes.c_int64)]


class DsaQueries(ctypes.Structure):
    _fields_ = [("num_queries", ctypes.c_int32), ("q_seq", ctypes.c_void_p),
                ("q_visible", ctypes.c_void_p), ("max_visible", ctypes.c_int32),
                ("total_visible", ctypes.c_int64)]


class DsaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}")
        self.status = status


_lib = None
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libdsa.so (raises if it has not been built).  DSA_LIB_PATH overrides the
    in-tree location."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or os.environ.get("DSA_LIB_PATH") or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           f"`python -m sparse_indexed_attention_amd.build`")
    lib = ctypes.CDLL(path)
    lib.dsa_indexer_topk_workspace_size.argtypes = [_I32, _I32, _I32]
    lib.dsa_indexer_topk_workspace_size.restype = _SZ
    lib.dsa_indexer_topk.argtypes = [_P, _I32, _P, _P, _I32, _P, _I32, _I32,
                                     ctypes.POINTER(DsaLayout), ctypes.POINTER(DsaQueries),
                                     _I32, _P, _P, _P, _SZ, _P]
    lib.dsa_indexer_topk.restype = _I32
    lib.dsa_indexer_topk_noalloc.argtypes = [_P, _I32, _P, _P, _I32, _P, _I32, _I32,
                                             ctypes.POINTER(DsaLayout), ctypes.POINTER(DsaQueries),
                                             _I32, _P, _P, _P]
    lib.dsa_indexer_topk_noalloc.restype = _I32
    lib.dsa_sparse_attn_workspace_size.argtypes = [_I32, _I32, _I32, _I32]
    lib.dsa_sparse_attn_workspace_size.restype = _SZ
    lib.dsa_sparse_attn.argtypes = [_P, _I32, _P, _I32, _I32, _I32, _I32, ctypes.c_float,
                                    ctypes.POINTER(DsaLayout), ctypes.POINTER(DsaQueries),
                                    _P, _I32, _P, _P, _P, _SZ, _P]
    lib.dsa_sparse_attn.restype = _I32
    lib.dsa_store_index_keys.argtypes = [_P, _I32, _I32, _P, _P, _I32, _P, _P]
    lib.dsa_store_index_keys.restype = _I32
    lib.dsa_store_kv.argtypes = [_P, _I32, _I32, _I32, _P, _P, _I32, _P]
    lib.dsa_store_kv.restype = _I32
    lib.dsa_status_string.argtypes = [_I32]
    lib.dsa_status_string.restype = ctypes.c_char_p
    lib.dsa_abi_version.argtypes = []
    lib.dsa_abi_version.restype = _I32
    lib.dsa_zigzag_ranges.argtypes = [ctypes.c_int64, _I32, _I32, _P]
    lib.dsa_zigzag_ranges.restype = _I32
    lib.dsa_indexer_prolog_workspace_size.argtypes = [_I32, _I32, _I32]
    lib.dsa_indexer_prolog_workspace_size.restype = _SZ
    lib.dsa_indexer_prolog.argtypes = [_P, _I32, _I32, _P, _P, ctypes.c_float, _I32, _I32,
                                       _P, _P, _P, _P, _P, _I32, _P, _P, _SZ, _P]
    lib.dsa_indexer_prolog.restype = _I32
    if hasattr(lib, "dsa_timeline_register"):     # the measurement build only
        lib.dsa_timeline_bytes.argtypes = []
        lib.dsa_timeline_bytes.restype = _SZ
        lib.dsa_timeline_register.argtypes = [_P, _SZ]
        lib.dsa_timeline_register.restype = _I32
    _lib = lib
    return lib


def timeline_bytes() -> int:
    """Size of the phase-stamp buffer (include/dsa_timeline.h); the measurement build
    libdsa_timeline.so only (load it with DSA_LIB_PATH)."""
    lib = load()
    if not hasattr(lib, "dsa_timeline_bytes"):
        raise RuntimeError("this libdsa has no phase stamps: load libdsa_timeline.so")
    return int(lib.dsa_timeline_bytes())


def timeline_register(buf) -> None:
    """Registers a device buffer of timeline_bytes() for the kernels' phase stamps
    (None stops recording); the measurement build only."""
    lib = load()
    if not hasattr(lib, "dsa_timeline_register"):
        raise RuntimeError("this libdsa has no phase stamps: load libdsa_timeline.so")
    nbytes = 0 if buf is None else buf.numel() * buf.element_size()
    st = lib.dsa_timeline_register(_ptr(buf), nbytes)
    if st != 0:
        raise DsaError("dsa_timeline_register", st)


# ------------------------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return DSA_F32
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return DSA_BF16
    if t.dtype in (torch.float8_e4m3fn, torch.uint8):
        return DSA_FP8_E4M3
    raise TypeError(f"unsupported tensor dtype {t.dtype}")


def _key_dtype(k_pool, k_scale) -> int:
    """Index-key storage: MXFP8 when the scales are bytes (E8M0, one per 32 dims), else the
    pool's own dtype (fp8 codes with fp32 per-token scales, bf16 or fp32)."""
    torch = _torch()
    if k_scale is not None and k_scale.dtype == torch.uint8:
        return DSA_MXFP8_E4M3
    return _dtype_code(k_pool)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def make_layout(block_table=None, block_size: int = 0, seq_stride: int = 0, num_seqs: int = 1,
                pool_rows: int = 0) -> DsaLayout:
    if block_table is not None:
        return DsaLayout(block_size, block_table.shape[1], block_table.data_ptr(), 0,
                         block_table.shape[0], pool_rows)
    return DsaLayout(0, 0, None, seq_stride, num_seqs, pool_rows)


def make_queries(q_seq, q_visible=None, max_visible: int = 0, total_visible: int = 0) -> DsaQueries:
    return DsaQueries(q_seq.shape[0], q_seq.data_ptr(),
                      None if q_visible is None else q_visible.data_ptr(), max_visible,
                      total_visible)


def zigzag_ranges(n_tokens: int, n_shards: int, shard: int):
    """((head_begin, head_end), (tail_begin, tail_end)) of one zigzag shard of a causal chunk
    (dsa_zigzag_ranges)."""
    r = (ctypes.c_int64 * 4)()
    st = load().dsa_zigzag_ranges(n_tokens, n_shards, shard, ctypes.cast(r, _P))
    if st != 0:
        raise DsaError("dsa_zigzag_ranges", st)
    return (r[0], r[1]), (r[2], r[3])


def indexer_workspace_bytes(num_queries: int, max_visible: int, top_k: int) -> int:
    return int(load().dsa_indexer_topk_workspace_size(num_queries, max_visible, top_k))


def sfa_workspace_bytes(num_queries: int, n_heads: int, top_k: int, d_v: int) -> int:
    return int(load().dsa_sparse_attn_workspace_size(num_queries, n_heads, top_k, d_v))


def zeroed_workspace(nbytes: int, device):
    """A zero-filled workspace buffer (the library keeps it zeroed between calls)."""
    return _torch().zeros(max(nbytes, 16), dtype=_torch().uint8, device=device)


def indexer_topk(q, head_w, k_pool, k_scale, layout: DsaLayout, q_seq, q_visible,
                 max_visible: int, top_k: int, *, out_idx=None, out_score=None,
                 want_score: bool = True, workspace=None, stream=None, total_visible: int = 0):
    """Fused lightning indexer + Top-K.  Shapes as in include/dsa.h:
    q [T, H_I, D_I] (float32 | bfloat16/int16 bits), head_w [T, H_I] float32,
    k_pool [rows, D_I] (float32 | bfloat16 bits | fp8 codes as uint8/float8_e4m3fn),
    k_scale [rows] float32 for fp8 keys, or uint8 [rows, D/32] E8M0 bytes for MXFP8 keys (the
    query is then quantized to MXFP8 inside the call).  Returns (idx [T, K] int32, score or
    None).  total_visible: the sum of q_visible if known on the host (sizes the launch), else
    0."""
    torch = _torch()
    lib = load()
    T, H, D = q.shape
    if out_idx is None:
        out_idx = torch.empty((T, top_k), dtype=torch.int32, device=q.device)
    if out_score is None and want_score:
        out_score = torch.empty((T, top_k), dtype=torch.float32, device=q.device)
    queries = make_queries(q_seq, q_visible, max_visible, total_visible)
    if workspace is None:
        workspace = zeroed_workspace(indexer_workspace_bytes(T, max_visible, top_k), q.device)
    st = lib.dsa_indexer_topk(_ptr(q), _dtype_code(q), _ptr(head_w), _ptr(k_pool),
                              _key_dtype(k_pool, k_scale), _ptr(k_scale), H, D, ctypes.byref(layout),
                              ctypes.byref(queries), top_k, _ptr(out_idx), _ptr(out_score),
                              _ptr(workspace), workspace.numel() * workspace.element_size(),
                              _stream(stream))
    if st != 0:
        raise DsaError("dsa_indexer_topk", st)
    return out_idx, out_score


def indexer_topk_noalloc(q, head_w, k_pool, k_scale, layout: DsaLayout, q_seq, q_visible,
                         max_visible: int, top_k: int, *, out_idx, out_score=None, stream=None,
                         total_visible: int = 0):
    """dsa_indexer_topk_noalloc: indexer_topk with the library's own device scratch array as
    the workspace (nothing is allocated by the call; out_idx, and out_score if wanted, are the
    caller's).  Returns (out_idx, out_score)."""
    lib = load()
    T, H, D = q.shape
    queries = make_queries(q_seq, q_visible, max_visible, total_visible)
    st = lib.dsa_indexer_topk_noalloc(_ptr(q), _dtype_code(q), _ptr(head_w), _ptr(k_pool),
                                      _key_dtype(k_pool, k_scale), _ptr(k_scale), H, D,
                                      ctypes.byref(layout), ctypes.byref(queries), top_k,
                                      _ptr(out_idx), _ptr(out_score), _stream(stream))
    if st != 0:
        raise DsaError("dsa_indexer_topk_noalloc", st)
    return out_idx, out_score


def sparse_attn(q, kv_pool, idx, layout: DsaLayout, q_seq, softmax_scale: float, d_v: int = 512,
                *, out=None, out_lse=None, want_lse: bool = True, workspace=None, stream=None):
    """Sparse Flash Attention.  q [T, H, d_qk] and kv_pool [rows, d_qk] share one dtype
    (float32, or bfloat16 / int16 bits), or kv_pool holds fp8 latent rows (uint8 [rows, 656],
    with bf16 q; the layout of DSA_KV_FP8_ROW_BYTES in include/dsa.h); idx [T, K] int32
    logical positions, -1 skipped.  Returns (out [T, H, d_v] in q's dtype, lse [T, H] float32
    or None)."""
    torch = _torch()
    lib = load()
    T, H, dqk = q.shape
    K = idx.shape[1]
    if out is None:
        out = torch.empty((T, H, d_v), dtype=q.dtype, device=q.device)
    if out_lse is None and want_lse:
        out_lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    queries = make_queries(q_seq, None, 0)
    if workspace is None:
        workspace = zeroed_workspace(sfa_workspace_bytes(T, H, K, d_v), q.device)
    st = lib.dsa_sparse_attn(_ptr(q), _dtype_code(q), _ptr(kv_pool), _dtype_code(kv_pool), H, dqk, d_v,
                             float(softmax_scale), ctypes.byref(layout), ctypes.byref(queries),
                             _ptr(idx), K, _ptr(out), _ptr(out_lse), _ptr(workspace),
                             workspace.numel() * workspace.element_size(), _stream(stream))
    if st != 0:
        raise DsaError("dsa_sparse_attn", st)
    return out, out_lse


def store_index_keys(k_new, slot, k_pool, k_scale=None, stream=None):
    """k_new [n, D] float32 -> k_pool rows slot[i] (int64) in k_pool's dtype; with uint8
    codes and uint8 k_scale [rows, D/32], MXFP8 (E8M0 byte per 32 dims)."""
    st = load().dsa_store_index_keys(_ptr(k_new), k_new.shape[0], k_new.shape[1], _ptr(slot),
                                     _ptr(k_pool), _key_dtype(k_pool, k_scale), _ptr(k_scale),
                                     _stream(stream))
    if st != 0:
        raise DsaError("dsa_store_index_keys", st)


_KEY_FORMATS = {"f32": 0, "bf16": 1, "fp8": 2, "mxfp8": 3}


def prolog_workspace_bytes(n_tokens: int, n_heads: int, head_dim: int) -> int:
    return int(load().dsa_indexer_prolog_workspace_size(n_tokens, n_heads, head_dim))


def indexer_prolog(x, w_proj, k_gain, eps: float, n_heads: int, head_dim: int, *, slot=None,
                   k_pool=None, k_scale=None, key_format: str = "bf16", want_k: bool = False,
                   q_out=None, w_out=None, k_out=None, workspace=None, stream=None):
    """dsa_indexer_prolog: x [T, d_x] bf16, w_proj [d_x, H*D + D + H] bf16, k_gain [D] float32
    -> (q [T, H, D] bf16, w [T, H] float32, k [T, D] float32 or None); with slot and k_pool
    the keys are also stored (k_pool's dtype as in store_index_keys).  Without a pool,
    key_format ("bf16", "fp8", "mxfp8", "f32") says which keys the query is made for (MXFP8
    keys: the query is MXFP8-quantized)."""
    torch = _torch()
    lib = load()
    T, d_x = x.shape
    if q_out is None:
        q_out = torch.empty((T, n_heads, head_dim), dtype=torch.bfloat16, device=x.device)
    if w_out is None:
        w_out = torch.empty((T, n_heads), dtype=torch.float32, device=x.device)
    if k_out is None and want_k:
        k_out = torch.empty((T, head_dim), dtype=torch.float32, device=x.device)
    kd = _key_dtype(k_pool, k_scale) if k_pool is not None else _KEY_FORMATS[key_format]
    if workspace is None:
        workspace = torch.empty(max(prolog_workspace_bytes(T, n_heads, head_dim), 16),
                                dtype=torch.uint8, device=x.device)
    st = lib.dsa_indexer_prolog(_ptr(x), T, d_x, _ptr(w_proj), _ptr(k_gain), float(eps), n_heads,
                                head_dim, _ptr(q_out), _ptr(w_out), _ptr(k_out), _ptr(slot),
                                _ptr(k_pool), kd, _ptr(k_scale), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(stream))
    if st != 0:
        raise DsaError("dsa_indexer_prolog", st)
    return q_out, w_out, k_out


def store_kv(kv_new, slot, kv_pool, stream=None):
    """kv_new [n, d_qk] (float32 | bf16 bits) -> kv_pool rows slot[i] in kv_pool's dtype
    (uint8 [rows, 656]: the fp8 latent rows of include/dsa.h, d_qk = 576)."""
    st = load().dsa_store_kv(_ptr(kv_new), _dtype_code(kv_new), kv_new.shape[0], kv_new.shape[1],
                             _ptr(slot), _ptr(kv_pool), _dtype_code(kv_pool), _stream(stream))
    if st != 0:
        raise DsaError("dsa_store_kv", st)
