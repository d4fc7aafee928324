// Host/device shared declarations: kernel parameter blocks, launch plans and launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dsa_common.hpp"

namespace dsa {

// ------------------------------------------------------------------ indexer + Top-K
constexpr int kIdxThreads = 256;
constexpr int kSplitMax = 2048;        // context positions scored by one workgroup
constexpr int kNSplitMax = 2048;       // context splits per query
constexpr int kMaxTopK = 2048;         // largest top_k
constexpr int kMinFastBlock = 32;      // smallest page size of the MFMA path (one page per 32-position group)
constexpr int kMinSplit = 512;         // shortest context split
constexpr int kCompactMaxT = 64;       // most queries of a compact indexer launch
constexpr int kGenericMaxHD = 8192;    // n_heads * head_dim on the reference path
constexpr int kGenericMaxHeads = 256;

enum { kDtF32 = 0, kDtBF16 = 1, kDtFP8 = 2, kDtMX = 3 };

struct IndexerPlan {
  int32_t grid;         // workgroups of the launch (a multi-query launch takes nsplit_max * ceil(T / 4))
  int32_t split;        // positions per context split (multiple of 64)
  int32_t nsplit_max;   // splits of the longest visible prefix (header rows per query)
  int32_t cap;          // candidates per split at most = min(split, top_k)
  int32_t rs;           // candidate slots per split: cap rounded up to 4
  int32_t compact;      // 1: the grid numbers only live splits (IndexerParams::compact)
  size_t off_counters, off_hdr, off_ckey, off_cpos, bytes;
};

struct IndexerParams {
  const void* q;
  const float* w;
  const void* k_pool;
  const float* k_scale;
  Layout L;
  const int32_t* q_seq;
  const int32_t* q_vis;
  int32_t T, H, D, K, max_visible;
  int32_t q_dtype, k_dtype;
  int32_t grid, split, nsplit_max, cap, rs;
  int32_t compact;      // items numbered over the live splits only (see the kernel)
  int32_t* out_idx;
  float* out_score;
  uint32_t* counters;   // [T]                  split arrivals per query (self-resetting)
  uint32_t* hdr;        // [T][nsplit_max][8]   emitted count, threshold key, key range
  uint32_t* cand_key;   // [T][nsplit_max][rs] one run of candidates per split: keys
  int32_t* cand_pos;    // [T][nsplit_max][rs] ... and positions
};

IndexerPlan plan_indexer_split(int32_t T, int32_t max_visible, int32_t top_k, int32_t split);
IndexerPlan plan_indexer(int32_t T, int32_t max_visible, int32_t top_k, int64_t total_visible);
size_t indexer_workspace_bytes(int32_t T, int32_t max_visible, int32_t top_k);
hipError_t launch_indexer(const IndexerParams& p, bool fast_path, hipStream_t stream);

// ------------------------------------------------------------------ sparse attention
constexpr int kSfaDqk = 576;
constexpr int kSfaDv = 512;
constexpr int kSfaRowF8 = 656;        // fp8 latent row: 512 codes, 64 bf16, 4 fp32 tile scales

struct SfaPlan {
  int32_t heads_per_wg;   // heads handled by one workgroup (fast path)
  int32_t n_hg;           // head groups
  int32_t rows_per_split; // selected rows per split (multiple of 32)
  int32_t nsplit;         // splits of top_k
  size_t off_zero, off_flags, off_part, off_ml, bytes;
};

struct SfaParams {
  const void* q;          // [T, H, d_qk]
  const void* kv;         // [rows, d_qk]
  Layout L;
  const int32_t* q_seq;
  const int32_t* idx;     // [T, K]
  int32_t T, H, dqk, dv, K;
  float scale;
  int32_t dtype;
  int32_t kv_dtype;       // dtype, or kDtFP8 for the tile-quantized latent rows
  int32_t heads_per_wg, n_hg, rows_per_split, nsplit;
  void* out;              // [T, H, d_v]
  float* lse;             // [T, H] or nullptr
  const void* zero;       // 16 zero bytes (source of the rows of absent positions)
  uint32_t* flags;        // [T][H/32][nsplit] bit c: head 32g + c to recompute by the reference method
  void* part_o;           // [T][H/32][nsplit] 32 KB blocks of fp16 partial outputs
  float* part_ml;         // [T][H][nsplit][2] exponent reference (exp2 domain), sum
};

SfaPlan plan_sfa(int32_t T, int32_t H, int32_t K, int32_t dv, bool fast_path);
hipError_t launch_sfa(const SfaParams& p, bool fast_path, hipStream_t stream);

// ------------------------------------------------------------------ cache writers
hipError_t launch_store_index_keys(const float* k_new, int32_t n, int32_t D, const int64_t* slot,
                                   void* k_pool, int32_t k_dtype, float* k_scale, hipStream_t s);
hipError_t launch_store_kv(const void* kv_new, int32_t src_dtype, int32_t n, int32_t dqk,
                           const int64_t* slot, void* kv_pool, int32_t pool_dtype, hipStream_t s);

// ------------------------------------------------------------------ indexer prolog
constexpr int kPrologMaxD = 1024;      // longest key (head_dim) of the prolog
constexpr int kMaxDevices = 64;

struct PrologParams {
  const float* y;         // [T, N] fp32 projections (workspace), N = H * D + D + H
  int32_t N, H, D;
  float eps;
  const float* gain;      // [D] RMSNorm gain of the key
  void* q_out;            // [T, H, D] bf16
  int32_t q_mx;           // quantize the query to MXFP8 (for MXFP8 keys)
  float* w_out;           // [T, H]
  float* k_out;           // [T, D] or nullptr
  const int64_t* slot;    // [T] key-pool rows, or nullptr with pool
  void* pool;             // key pool or nullptr (no store)
  int32_t k_dt;
  float* k_scale;
};

// rocBLAS GEMM then the epilogue; *blas_status is the rocblas_status when that failed
hipError_t run_prolog(const void* x, int32_t T, int32_t d_x, const void* w_proj,
                      const PrologParams& p, hipStream_t stream, int* blas_status);

}  // namespace dsa
