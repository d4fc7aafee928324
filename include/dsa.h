/*
 * dsa.h - C ABI of the DSA sparse-attention hot path on AMD Instinct MI355X (gfx950).
 *
 * The path has two stages ("Day0 Adaptation and Sparse Attention Optimization for
 * Long-Sequence LLM Inference", section 4: index generation, then sparse read):
 *
 *   dsa_indexer_topk  - the lightning indexer fused with Top-K.  For every query it scores
 *                       each visible cached position with per-head dot products, ReLU and a
 *                       head-weighted sum, and keeps the K best positions.  It reads the
 *                       paged index-key cache directly and writes only the index list
 *                       ("Large Model Inference Acceleration: Day-0 Adaptation...", section
 *                       1.1; "Day0 Adaptation and Performance Optimization for Novel
 *                       Long-Sequence Reasoning Models", section 3).
 *   dsa_sparse_attn   - Sparse Flash Attention: gathers the selected rows of the paged MLA
 *                       latent cache and computes softmax attention over them only (same
 *                       sections; the latent row is the key, its first d_v columns the value).
 *
 * plus the cache writers that fill the pools in this layout.
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers unless marked (host).  Structs are passed by host pointer.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null stream).  They never
 *     allocate or free device memory and never synchronize the host.
 *   - Validation happens on the host before anything is launched.  On any error the call
 *     returns a non-zero status and launches nothing, so outputs are untouched.  A failed
 *     launch returns DSA_ERR_HIP.  Device-side contents (block-table entries, per-query
 *     lengths beyond `max_visible`, NaN/Inf values) are the caller's contract and are not
 *     checked on the device.
 *   - Every device pointer must be 16-byte aligned (DSA_ERR_ALIGN otherwise).  Pool rows are
 *     dense (row stride = row width).
 *   - The library keeps no device memory.  Its only process-wide state is set once and never
 *     changed afterwards: the planners' measurement overrides, read from the environment at
 *     the first planned call (DSA_INDEXER_TARGET_WG, DSA_INDEXER_MQ, DSA_SFA_HPW,
 *     DSA_SFA_SPLITS; unset means the planners' own choice), and for dsa_indexer_prolog one
 *     rocBLAS handle per device, created at that device's first call under a lock.
 *   - Two calls that share a workspace must not run concurrently.
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_ABI_VERSION 3

typedef enum {
  DSA_OK = 0,
  DSA_ERR_NULL = 1,        /* a required pointer is NULL                                   */
  DSA_ERR_SHAPE = 2,       /* a size is out of range or inconsistent                       */
  DSA_ERR_DTYPE = 3,       /* a dtype is not accepted for that argument                     */
  DSA_ERR_UNSUPPORTED = 4, /* valid in principle, not built (e.g. head_dim or top_k too large) */
  DSA_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than the *_workspace_size query      */
  DSA_ERR_ALIGN = 6,       /* a device pointer is not 16-byte aligned                       */
  DSA_ERR_HIP = 7,         /* a HIP runtime call or kernel launch failed                    */
  DSA_ERR_BLAS = 8         /* the library GEMM (rocBLAS) failed                             */
} dsa_status;

typedef enum {
  DSA_F32 = 0,             /* IEEE binary32                                                 */
  DSA_BF16 = 1,            /* bfloat16 bits in uint16                                       */
  DSA_FP8_E4M3 = 2,        /* OCP fp8 e4m3 "fn" (no infinities, max 448), one byte          */
  DSA_MXFP8_E4M3 = 3       /* OCP MXFP8: e4m3 codes, one E8M0 scale byte per 32 elements    */
} dsa_dtype;

/* Paged-cache layout, shared by every pool of a call (index keys, their scales, latent KV).
 *   block_table != NULL: position s of sequence b is pool row
 *       block_table[b * max_blocks_per_seq + (s / block_size)] * block_size + s % block_size
 *   block_table == NULL: sequences are contiguous: row = b * seq_stride + s.
 * block_size is a power of two between 1 and 65536 when a block table is given.  Block-table
 * columns past the blocks a query can see are never read.  pool_rows (host) is the number of
 * rows in each pool; it bounds contiguous layouts and is otherwise informational. */
typedef struct {
  int32_t block_size;
  int32_t max_blocks_per_seq;
  const int32_t* block_table;   /* [num_seqs, max_blocks_per_seq] or NULL                   */
  int64_t seq_stride;           /* rows between sequences when block_table == NULL           */
  int32_t num_seqs;             /* (host) number of sequences the table / stride covers      */
  int64_t pool_rows;            /* (host)                                                     */
} dsa_layout;

/* Which sequence each query belongs to and how much of it the query sees.  Query t sees
 * positions [0, q_visible[t]) of sequence q_seq[t]: causal, its own position included.  A
 * decode query sees its whole sequence; query i of a chunk of new tokens appended to a
 * prefix of P tokens sees P + i + 1.  max_visible (host) must be >= every q_visible[t]; it
 * sizes the launch so that the host never reads device memory.  total_visible (host,
 * optional) is the sum of q_visible over the queries when the caller knows it, else 0; the
 * indexer then sizes its context splits to the real total instead of T * max_visible.  It
 * only steers the launch: a wrong value costs time, never correctness (it is clamped to
 * [max_visible, T * max_visible]). */
typedef struct {
  int32_t num_queries;          /* T >= 1                                                     */
  const int32_t* q_seq;         /* [T], 0 <= q_seq[t] < num_seqs                              */
  const int32_t* q_visible;     /* [T], 1 <= q_visible[t] <= max_visible                      */
  int32_t max_visible;          /* (host) 1 <= max_visible <= DSA_MAX_CONTEXT                 */
  int64_t total_visible;        /* (host) sum of q_visible, or 0 if unknown                   */
} dsa_queries;

#define DSA_MAX_CONTEXT (1 << 22)  /* longest visible prefix a query may have (4M tokens)    */
#define DSA_MAX_TOPK 2048

/* FP8 latent KV row (kv_dtype / pool_dtype DSA_FP8_E4M3, MLA geometry d_qk = 576, d_v = 512):
 * the SFA cache quantized per token and per tile of 128 elements ("Day0 Adaptation and
 * Performance Optimization for Novel Long-Sequence Reasoning Models", section 4; "Day0
 * Adaptation and Sparse Attention Optimization for Long-Sequence LLM Inference", section 5;
 * "Optimizing and Deploying Ultra-Long Sequence Inference Architectures", section II; "Large
 * Model Inference Acceleration: Day-0 Adaptation...", section 2.2).  One row is 656 bytes:
 *   bytes [0, 512)    e4m3 codes of columns 0 .. 511, four tiles of 128 columns;
 *   bytes [512, 640)  columns 512 .. 575 (the rope part) as bf16, little-endian;
 *   bytes [640, 656)  the four tiles' scales as fp32.
 * Column j < 512 is code_j * scale[j / 128].  A tile's scale is the smallest power of two
 * 2^e (-126 <= e <= 127) with max |x| <= 448 * 2^e over the tile (1 for an all-zero tile), so
 * x / scale never saturates and every dequantized value is exact in bf16. */
#define DSA_KV_FP8_ROW_BYTES 656

/* ---------------------------------------------------------------------------------------
 * Lightning indexer + Top-K
 *
 * For query t (sequence b = q_seq[t], V = q_visible[t]) and every position s < V:
 *     x[h]   = sum_d q[t, h, d] * key(s)[d]          h < n_heads, d < head_dim
 *     S[s]   = sum_h head_w[t, h] * max(x[h], 0)
 * with key(s) = k_pool row of s, times k_scale[row] when k_dtype is FP8_E4M3.  One key
 * vector per token serves every indexer head.  With k_dtype MXFP8_E4M3 (the pages' group-32
 * MXFP8 quantization of index Q and K: "Day0 Adaptation and Performance Optimization for
 * Novel Long-Sequence Reasoning Models", section 4; "Optimizing and Deploying Ultra-Long
 * Sequence Inference Architectures", section II) key(s)[d] = code * 2^(e - 127) with e the
 * row's scale byte of group d / 32, and the query is quantized the same way inside the call,
 * per head and group of 32 dims (E8M0 byte = floor(log2 max|q|) - 8 + 127 clamped to
 * [0, 254], 0 for an all-zero group; code = e4m3(q * 2^(127 - byte)), nearest even,
 * saturated), before the dot products.  Scores are fp32.  The call keeps the
 * K_eff = min(top_k, V) largest scores, the lower position first among equal scores (-0 and
 * +0 compare equal), and writes their positions (logical positions within the sequence, not
 * pool rows) to out_idx[t, 0 .. K_eff) in ascending position order, then -1 up to top_k.
 * out_score (optional) receives the matching fp32 scores (0 after K_eff).
 *
 * Accepted inputs
 *   q:      [T, n_heads, head_dim], q_dtype F32 or BF16
 *   head_w: [T, n_heads] fp32 (any global scale folded in by the caller)
 *   k_pool: [pool_rows, head_dim], k_dtype F32, BF16, FP8_E4M3 or MXFP8_E4M3 (codes)
 *   k_scale:[pool_rows] fp32 for FP8_E4M3; for MXFP8_E4M3 the E8M0 bytes
 *           [pool_rows, head_dim / 32] (passed through this pointer); ignored otherwise
 *   1 <= n_heads * head_dim <= 8192, head_dim % 8 == 0 (% 32 for MXFP8_E4M3),
 *   1 <= top_k <= DSA_MAX_TOPK.
 * The fast path (MFMA scoring) runs for q BF16, keys BF16, FP8_E4M3 or MXFP8_E4M3, n_heads
 * 64, head_dim 128 and a contiguous layout or block_size >= 32; fp8 codes are widened to bf16
 * exactly (with their scale where it is a power of two) and summed in fp32.  Every other
 * accepted combination runs a reference path that scores in fp64.
 *
 * workspace: dsa_indexer_topk_workspace_size(...) bytes.  It MUST be zero-filled before its
 * first use; every call leaves it zero-filled again where that matters (the per-query arrival
 * counters, kept in a block of their own at its start for up to 8192 queries), so one buffer
 * can be reused across calls of any size up to the one it was sized for.
 * --------------------------------------------------------------------------------------- */
size_t dsa_indexer_topk_workspace_size(int32_t num_queries, int32_t max_visible, int32_t top_k);

dsa_status dsa_indexer_topk(const void* q, dsa_dtype q_dtype, const float* head_w,
                            const void* k_pool, dsa_dtype k_dtype, const float* k_scale,
                            int32_t n_heads, int32_t head_dim,
                            const dsa_layout* layout, const dsa_queries* queries,
                            int32_t top_k, int32_t* out_idx, float* out_score,
                            void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * dsa_indexer_topk_noalloc: dsa_indexer_topk for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * arguments, results and errors are those of dsa_indexer_topk without the workspace: the call
 * uses a scratch array of DSA_NOALLOC_SCRATCH_BYTES bytes that the library holds in device
 * memory (one per device, from the device's first use of the library until the process
 * ends) and calls no allocator.
 *   - A call whose plan needs more scratch than that returns DSA_ERR_WORKSPACE and launches
 *     nothing (decode batches fit: 8 queries of 128K, 32 of 32K or one of 4M positions need
 *     under 9 MB; a prefill chunk of thousands of queries does not: use dsa_indexer_topk).
 *   - The first call on a device looks up the array's device address and enqueues a kernel
 *     that zeroes it on `stream` before the indexer (a failure there returns DSA_ERR_HIP).
 *   - Every call on one device shares the array: calls that overlap on one device (other
 *     streams, other host threads) race and must be serialized by the caller.
 * --------------------------------------------------------------------------------------- */
#define DSA_NOALLOC_SCRATCH_BYTES (32u << 20)

dsa_status dsa_indexer_topk_noalloc(const void* q, dsa_dtype q_dtype, const float* head_w,
                                    const void* k_pool, dsa_dtype k_dtype, const float* k_scale,
                                    int32_t n_heads, int32_t head_dim,
                                    const dsa_layout* layout, const dsa_queries* queries,
                                    int32_t top_k, int32_t* out_idx, float* out_score,
                                    void* stream);

/* ---------------------------------------------------------------------------------------
 * Sparse Flash Attention over the selected rows of the MLA latent cache
 *
 * For query t (sequence b = q_seq[t]) let J be the entries of idx[t, 0 .. top_k) that are
 * not -1 (positions in sequence b; repeated entries count once per occurrence) and R_j the
 * kv_pool row of position j.  For every head h < n_heads:
 *     z_j = softmax_scale * dot(q[t, h, 0 .. d_qk), R_j[0 .. d_qk))
 *     out[t, h, :] = sum_j softmax(z)_j * R_j[0 .. d_v)
 *     out_lse[t, h] = log(sum_j exp(z_j))           (natural log; optional)
 * With J empty: out = 0 and out_lse = -inf.
 *
 * dtype applies to q and out: BF16 (fp32 accumulation, MFMA) or F32 (reference mode, fp32
 * throughout).  kv_dtype is the storage of kv_pool: the same as dtype, or FP8_E4M3 with
 * dtype BF16 for the tile-quantized rows above (d_qk = 576 and d_v = 512 only; R_j is the
 * dequantized row).  d_qk % 64 == 0, d_v % 64 == 0, d_v <= d_qk <= 1024,
 * 1 <= n_heads <= 1024; the BF16 path needs n_heads % 32 == 0, d_qk = 576 and d_v = 512 (the
 * MLA latent geometry), other shapes run the reference path.  idx entries must be -1 or
 * positions whose rows exist; they need not be sorted.
 * workspace: dsa_sparse_attn_workspace_size(...) bytes, zero-filled before first use, left
 * zero-filled where that matters.
 * --------------------------------------------------------------------------------------- */
size_t dsa_sparse_attn_workspace_size(int32_t num_queries, int32_t n_heads, int32_t top_k,
                                      int32_t d_v);

dsa_status dsa_sparse_attn(const void* q, dsa_dtype dtype, const void* kv_pool,
                           dsa_dtype kv_dtype, int32_t n_heads, int32_t d_qk, int32_t d_v,
                           float softmax_scale,
                           const dsa_layout* layout, const dsa_queries* queries,
                           const int32_t* idx, int32_t top_k, void* out, float* out_lse,
                           void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * Cache writers (outside the timed hot path; they produce the layout the two calls read).
 *
 * dsa_store_index_keys: k_new [n_tokens, head_dim] fp32 -> pool rows slot[i].
 *   k_dtype F32 / BF16: stored as is / rounded to nearest even.
 *   k_dtype FP8_E4M3: per-token quantization, as in the quantized indexer path ("Day0
 *   Adaptation and Performance Optimization for Novel Long-Sequence Reasoning Models",
 *   section 3) with one fp32 scale per token: scale = max_d |k| / 448 (1 if the token is
 *   all zero), code = fp8(k / scale) rounded to nearest even, saturating at +-448; the scale
 *   goes to k_scale[slot[i]].
 *   k_dtype MXFP8_E4M3 (head_dim % 32 == 0): per group of 32 dims the E8M0 byte and codes
 *   defined under dsa_indexer_topk; the bytes go to ((uint8_t*)k_scale)[slot[i] * head_dim / 32
 *   + group].
 * dsa_store_kv: kv_new [n_tokens, d_qk] (src_dtype F32 or BF16) -> kv_pool rows slot[i] in
 *   pool_dtype (F32 or BF16; F32 -> BF16 rounds to nearest even), or FP8_E4M3 for the
 *   tile-quantized rows of DSA_KV_FP8_ROW_BYTES bytes (d_qk = 576): per tile the scale
 *   defined there, code = fp8(x / scale) rounded to nearest even; the rope columns are
 *   rounded to bf16 (nearest even) or copied.
 * slot[i] is the pool row (block * block_size + offset) of token i; rows must be distinct.
 * --------------------------------------------------------------------------------------- */
dsa_status dsa_store_index_keys(const float* k_new, int32_t n_tokens, int32_t head_dim,
                                const int64_t* slot, void* k_pool, dsa_dtype k_dtype,
                                float* k_scale, void* stream);

dsa_status dsa_store_kv(const void* kv_new, dsa_dtype src_dtype, int32_t n_tokens, int32_t d_qk,
                        const int64_t* slot, void* kv_pool, dsa_dtype pool_dtype, void* stream);

/* ---------------------------------------------------------------------------------------
 * dsa_indexer_prolog: the indexer's inputs for n_tokens new tokens, from their hidden vectors
 * ("Day0 Adaptation and Performance Optimization for Novel Long-Sequence Reasoning Models",
 * section 3; "Large Model Inference Acceleration: Day-0 Adaptation...", section 1.2;
 * "Optimizing and Deploying Ultra-Long Sequence Inference Architectures", section I: query
 * projection, key normalization, query quantization, head-weight projection), and the key's
 * store into the paged key pool.  With H = n_heads, D = head_dim, N = H * D + D + H:
 *     Y = x w_proj                          fp32 sums of bf16 products (one library GEMM)
 *     q_out[t, h, d] = Y[t, h * D + d]      bf16, nearest even; for k_dtype MXFP8_E4M3 the
 *                                           MXFP8 group-32 quantization of Y's query part
 *                                           (defined under dsa_indexer_topk), dequantized
 *     k[t, d]  = Y[t, H*D + d] / sqrt(mean_d Y[t, H*D + d]^2 + eps) * k_gain[d]
 *     w_out[t, h] = Y[t, H*D + D + h]       fp32
 * and k[t] is written to k_pool row slot[t] as dsa_store_index_keys writes it (k_dtype F32,
 * BF16, FP8_E4M3 with k_scale, or MXFP8_E4M3 with its scale bytes in k_scale).
 *   x:       [n_tokens, d_x] bf16 (device)
 *   w_proj:  [d_x, N] bf16 row-major (device): columns [0, H*D) the query, head-major, then
 *            D key columns, then H head-weight columns
 *   k_gain:  [D] fp32 (device); eps >= 0
 *   q_out:   [n_tokens, H, D] bf16; w_out: [n_tokens, H] fp32; k_out: [n_tokens, D] fp32 or
 *            NULL (the normalized keys before their storage rounding)
 *   slot, k_pool, k_scale: the store; slot and k_pool both NULL skips it
 *   1 <= head_dim <= 1024 (% 32 == 0 for MXFP8_E4M3), n_heads >= 1, n_heads * head_dim <=
 *   65534 * 2048, d_x >= 1, 1 <= n_tokens <= 2^20.  All buffers are the caller's and stay so.
 * workspace: dsa_indexer_prolog_workspace_size(...) bytes (any contents).  The call
 * enqueues the GEMM and one kernel on `stream` and returns; the library keeps one rocBLAS
 * handle per device (created on first use) and serializes only the enqueueing of calls.
 * Errors: DSA_ERR_NULL, DSA_ERR_SHAPE, DSA_ERR_DTYPE, DSA_ERR_UNSUPPORTED (beyond those sizes),
 * DSA_ERR_WORKSPACE, DSA_ERR_ALIGN, DSA_ERR_BLAS (rocBLAS refused or failed), DSA_ERR_HIP.
 * --------------------------------------------------------------------------------------- */
size_t dsa_indexer_prolog_workspace_size(int32_t n_tokens, int32_t n_heads, int32_t head_dim);

dsa_status dsa_indexer_prolog(const void* x, int32_t n_tokens, int32_t d_x, const void* w_proj,
                              const float* k_gain, float eps, int32_t n_heads, int32_t head_dim,
                              void* q_out, float* w_out, float* k_out, const int64_t* slot,
                              void* k_pool, dsa_dtype k_dtype, void* k_scale, void* workspace,
                              size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * dsa_zigzag_ranges: the token ranges of one shard of a causal chunk under the zigzag
 * head-tail layout ("Day0 Adaptation and Performance Optimization for Novel Long-Sequence
 * Reasoning Models", section 5; "Large Model Inference Acceleration: Day-0 Adaptation...",
 * section 3.1; "Optimizing and Deploying Ultra-Long Sequence Inference Architectures",
 * section 3.2).  A chunk of n_tokens new tokens (token i sees prefix + i + 1 positions, so
 * later tokens cost more) is cut into 2 * n_shards segments, segment s being
 * [floor(s * n_tokens / (2 n_shards)), floor((s + 1) * n_tokens / (2 n_shards))); shard g
 * takes segment g (its head range) and segment 2 n_shards - 1 - g (its tail range), which
 * pairs short and long histories.  Running each shard's queries (dsa_indexer_topk and
 * dsa_sparse_attn over just those rows of q, head_w, q_seq and q_visible) and putting the
 * rows back in token order gives the unsharded result.
 *   ranges (host, 4 int64): written with {head_begin, head_end, tail_begin, tail_end}.
 * Host-only arithmetic: no device is touched.  Errors: DSA_ERR_NULL (ranges NULL),
 * DSA_ERR_SHAPE (n_tokens < 0, n_shards < 1, shard outside [0, n_shards)).
 * --------------------------------------------------------------------------------------- */
dsa_status dsa_zigzag_ranges(int64_t n_tokens, int32_t n_shards, int32_t shard, int64_t* ranges);

/* Human-readable name of a status (static storage, never NULL). */
const char* dsa_status_string(dsa_status status);

/* DSA_ABI_VERSION of the built library. */
int32_t dsa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H_ */
