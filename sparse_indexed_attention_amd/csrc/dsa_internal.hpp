// Host/device shared declarations: kernel parameter blocks, launch plans and launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dsa_common.hpp"

namespace dsa {

// Measurement overrides of the launch planners, read from the environment once per process
// (at the first call that plans a launch) and constant afterwards; 0 means "planner's choice".
//   DSA_INDEXER_TARGET_WG  indexer workgroups aimed for         DSA_INDEXER_MQ=0  no multi-query tiles
//   DSA_SFA_HPW            heads per attention workgroup        DSA_SFA_SPLITS    index-list slices
struct PlanOverrides {
  int64_t indexer_target_wg;
  int32_t indexer_mq_off;
  int32_t sfa_hpw;
  int64_t sfa_splits;
};
const PlanOverrides& plan_overrides();

// ------------------------------------------------------------------ phase stamps
// The measurement build of the library (-DDSA_TIMELINE, libdsa_timeline.so; never libdsa.so)
// records when each workgroup ends each phase of its work: thread 0 writes the 100 MHz
// constant clock (s_memrealtime) into a device buffer the caller registers
// (dsa_timeline_register), laid out as u64 [kernel][workgroup][slot]; a slot a workgroup
// never reaches keeps the caller's zero.  Without the macro the stamps compile to nothing and
// the parameter blocks' `tl` pointer stays null.
constexpr int kTlMaxWg = 4096, kTlSlots = 32;
enum { kTlIndexer = 0, kTlSfa = 1, kTlCombine = 2, kTlKernels = 3 };
// slots of the indexer (single-query items): start, scored, candidates stored, arrived, and
// for the merging workgroup headers read, list staged, K-th key found, output written; the
// item (t << 16 | j) and whether it merged go to kTlItem and kTlLast
enum { kTlStart = 0, kTlScored = 1, kTlEmitted = 2, kTlArrived = 3, kTlHeaders = 4,
       kTlStaged = 5, kTlKth = 6, kTlMerged = 7, kTlItem = 14, kTlLast = 15 };
// finer indexer slots: the split's cut chosen, its candidate and header stores issued (before
// the drain that kTlEmitted ends), and in the merge the bin of the K-th key found
enum { kTlCut = 16, kTlStoresIssued = 17, kTlKthBin = 18 };
// slots of the attention kernels: start, rows resolved, first tiles and query rows landed,
// query fragments in registers, last tile done, outputs or partials written
enum { kTlRows = 1, kTlFirstTile = 2, kTlQueries = 3, kTlLoopDone = 4, kTlWritten = 5 };
// both: wave 0's shader-clock cycles waiting for loads and computing in the main loop, and its
// steps (key groups or tile pairs)
enum { kTlWaitCycles = 8, kTlComputeCycles = 9, kTlSteps = 10 };
// both: the shader clock (s_memtime) at the start and at the end of the main loop's phase
// (indexer: split scored; attention: last tile done), for the clock rate; indexer: the wall
// clock when the scoring loop starts
enum { kTlClockStart = 11, kTlClockEnd = 12, kTlLoopStart = 13 };
// attention (128-head kernel): wave 0's shader-clock cycles issuing the next tile's loads
enum { kTlIssueCycles = 19 };
uint64_t* timeline_buffer();   // the registered buffer (measurement build), else nullptr
#ifdef DSA_TIMELINE
__device__ __forceinline__ void tl_put(uint64_t* tl, int kernel, int slot, uint64_t v) {
  const int wg = blockIdx.x + blockIdx.y * gridDim.x;
  if (tl != nullptr && threadIdx.x == 0 && wg < kTlMaxWg)
    tl[((size_t)kernel * kTlMaxWg + wg) * kTlSlots + slot] = v;
}
__device__ __forceinline__ void tl_stamp(uint64_t* tl, int kernel, int slot) {
  tl_put(tl, kernel, slot, __builtin_amdgcn_s_memrealtime());
}
__device__ __forceinline__ void tl_clock(uint64_t* tl, int kernel, int slot) {
  tl_put(tl, kernel, slot, __builtin_amdgcn_s_memtime());
}
// Shader-clock cycles (s_memtime) wave 0 spends waiting for a loop's loads, computing and
// issuing loads, over the loop's steps: slots kTlWaitCycles, kTlComputeCycles, kTlIssueCycles
// and kTlSteps.  Each of waited(), computed() and issued() counts the cycles since the last
// mark or count.
struct TlCycles {
  uint64_t w = 0, c = 0, s = 0, t = 0;
  __device__ __forceinline__ void mark() { t = __builtin_amdgcn_s_memtime(); }
  __device__ __forceinline__ uint64_t lap() {
    const uint64_t n = __builtin_amdgcn_s_memtime(), d = n - t;
    t = n;
    return d;
  }
  __device__ __forceinline__ void waited() { w += lap(); }
  __device__ __forceinline__ void computed() { c += lap(); }
  __device__ __forceinline__ void issued() { s += lap(); }
  __device__ __forceinline__ void put(uint64_t* tl, int kernel, int steps) {
    if (threadIdx.x < 64) {
      tl_put(tl, kernel, kTlWaitCycles, w);
      tl_put(tl, kernel, kTlComputeCycles, c);
      if (s != 0) tl_put(tl, kernel, kTlIssueCycles, s);
      tl_put(tl, kernel, kTlSteps, (uint64_t)steps);
    }
  }
};
#else
__device__ __forceinline__ void tl_put(uint64_t*, int, int, uint64_t) {}
__device__ __forceinline__ void tl_stamp(uint64_t*, int, int) {}
__device__ __forceinline__ void tl_clock(uint64_t*, int, int) {}
struct TlCycles {
  __device__ __forceinline__ void mark() {}
  __device__ __forceinline__ void waited() {}
  __device__ __forceinline__ void computed() {}
  __device__ __forceinline__ void issued() {}
  __device__ __forceinline__ void put(uint64_t*, int, int) {}
};
#endif

// ------------------------------------------------------------------ indexer + Top-K
constexpr int kIdxThreads = 256;
constexpr int kSplitMax = 2048;        // context positions scored by one workgroup
constexpr int kNSplitMax = 2048;       // context splits per query
constexpr int kMaxTopK = 2048;         // largest top_k
constexpr int kMinFastBlock = 32;      // smallest page size of the MFMA path (one page per 32-position group)
constexpr int kMinSplit = 512;         // shortest context split
constexpr int kCompactMaxT = 64;       // most queries of a compact indexer launch
// The workspace starts with the queries' arrival counters, words that are zero between calls.
// Every layout puts the rest at kCtrlBytes or later (at 4 T bytes for more queries than fit),
// so no shape's headers or candidates land on another shape's counters, and one buffer serves
// calls of any shape it is large enough for.
constexpr size_t kCtrlBytes = 32768;
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
  size_t off_counters, off_hdr, off_ckey, off_cpos, off_qmx, bytes;
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
  uint16_t* q_mx;       // [T][64][128] MXFP8 keys: the queries quantized once per call (their
                        // dequantized values, exact in bf16), written before the main kernel
  uint64_t* tl;         // phase stamps (measurement build only), else nullptr
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
  int32_t decode64;       // 1: the 64-head, four-wave decode kernel
  int32_t dim_waves;      // waves of an attention workgroup, each owning d_v / dim_waves dims
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
  int32_t decode64, dim_waves;   // as in SfaPlan
  void* out;              // [T, H, d_v]
  float* lse;             // [T, H] or nullptr
  const void* zero;       // 16 zero bytes (source of the rows of absent positions)
  uint32_t* flags;        // [T][H/32][nsplit] bit c: head 32g + c to recompute by the reference method
  void* part_o;           // [T][H/32][nsplit] 32 KB blocks of fp16 partial outputs
  float* part_ml;         // [T][H][nsplit][2] exponent reference (exp2 domain), sum
  uint64_t* tl;           // phase stamps (measurement build only), else nullptr
};

SfaPlan plan_sfa(int32_t T, int32_t H, int32_t K, int32_t dv, bool fast_path, bool kv_fp8);
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
