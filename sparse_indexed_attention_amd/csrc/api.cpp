// C ABI of the DSA hot path: host-side validation, launch planning and dispatch.
// Nothing here reads device memory or synchronizes; errors are returned before any launch.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>

#include "../../include/dsa.h"
#include "../../include/dsa_timeline.h"
#include "dsa_internal.hpp"

namespace {

using namespace dsa;

bool misaligned(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

int log2i(int64_t x) {
  int l = 0;
  while ((int64_t(1) << l) < x) ++l;
  return l;
}

dsa_status check_layout(const dsa_layout* L, const dsa_queries* Q, bool need_visible) {
  if (!L || !Q) return DSA_ERR_NULL;
  if (!Q->q_seq || (need_visible && !Q->q_visible)) return DSA_ERR_NULL;
  if (Q->num_queries < 1 || Q->num_queries > 65535) return DSA_ERR_SHAPE;
  if (L->num_seqs < 1) return DSA_ERR_SHAPE;
  if (need_visible && (Q->max_visible < 1 || Q->max_visible > DSA_MAX_CONTEXT))
    return DSA_ERR_SHAPE;
  if (misaligned(L->block_table) || misaligned(Q->q_seq) || misaligned(Q->q_visible))
    return DSA_ERR_ALIGN;
  if (L->block_table) {
    if (!is_pow2(L->block_size) || L->block_size > 65536) return DSA_ERR_SHAPE;
    if (L->max_blocks_per_seq < 1) return DSA_ERR_SHAPE;
    if (need_visible &&
        (int64_t)L->max_blocks_per_seq * L->block_size < (int64_t)Q->max_visible)
      return DSA_ERR_SHAPE;
  } else {
    if (L->seq_stride < 1) return DSA_ERR_SHAPE;
    if (need_visible && L->seq_stride < Q->max_visible) return DSA_ERR_SHAPE;
    if (L->pool_rows < (int64_t)(L->num_seqs - 1) * L->seq_stride + (need_visible ? Q->max_visible : 1))
      return DSA_ERR_SHAPE;
  }
  return DSA_OK;
}

Layout make_layout(const dsa_layout* L) {
  Layout d{};
  d.bt = L->block_table;
  d.bt_stride = L->max_blocks_per_seq;
  d.bs_log2 = L->block_table ? log2i(L->block_size) : 0;
  d.seq_stride = L->seq_stride;
  return d;
}

bool indexer_fast(dsa_dtype q_dtype, dsa_dtype k_dtype, int32_t H, int32_t D,
                  const dsa_layout* L) {
  return q_dtype == DSA_BF16 &&
         (k_dtype == DSA_BF16 || k_dtype == DSA_FP8_E4M3 || k_dtype == DSA_MXFP8_E4M3) && H == 64 &&
         D == 128 && (!L->block_table || L->block_size >= kMinFastBlock);
}

bool sfa_fast(dsa_dtype dtype, int32_t H, int32_t dqk, int32_t dv) {
  return dtype == DSA_BF16 && dqk == kSfaDqk && dv == kSfaDv && H % 32 == 0;
}

}  // namespace

namespace dsa {
const PlanOverrides& plan_overrides() {
  static const PlanOverrides o = [] {
    PlanOverrides v{};
    auto num = [](const char* name) -> int64_t {
      const char* e = std::getenv(name);
      return e ? std::atoll(e) : 0;
    };
    v.indexer_target_wg = num("DSA_INDEXER_TARGET_WG");
    const char* mq = std::getenv("DSA_INDEXER_MQ");
    v.indexer_mq_off = mq && std::atoi(mq) == 0;
    v.sfa_hpw = (int32_t)num("DSA_SFA_HPW");
    v.sfa_splits = num("DSA_SFA_SPLITS");
    return v;
  }();
  return o;
}
// The registered stamp buffer of the measurement build; libdsa.so has none.
#ifdef DSA_TIMELINE
static uint64_t* g_timeline = nullptr;
uint64_t* timeline_buffer() { return g_timeline; }
#else
uint64_t* timeline_buffer() { return nullptr; }
#endif
}  // namespace dsa

extern "C" {

#ifdef DSA_TIMELINE
size_t dsa_timeline_bytes(void) { return (size_t)kTlKernels * kTlMaxWg * kTlSlots * sizeof(uint64_t); }

dsa_status dsa_timeline_register(void* buf, size_t bytes) {
  if (buf && bytes < dsa_timeline_bytes()) return DSA_ERR_WORKSPACE;
  if (misaligned(buf)) return DSA_ERR_ALIGN;
  g_timeline = static_cast<uint64_t*>(buf);
  return DSA_OK;
}
#endif

size_t dsa_indexer_topk_workspace_size(int32_t num_queries, int32_t max_visible, int32_t top_k) {
  if (num_queries < 1 || max_visible < 1 || max_visible > DSA_MAX_CONTEXT || top_k < 1) return 0;
  return indexer_workspace_bytes(num_queries, max_visible, top_k);
}

dsa_status dsa_indexer_topk(const void* q, dsa_dtype q_dtype, const float* head_w,
                            const void* k_pool, dsa_dtype k_dtype, const float* k_scale,
                            int32_t n_heads, int32_t head_dim, const dsa_layout* layout,
                            const dsa_queries* queries, int32_t top_k, int32_t* out_idx,
                            float* out_score, void* workspace, size_t workspace_bytes,
                            void* stream) {
  if (!q || !head_w || !k_pool || !out_idx) return DSA_ERR_NULL;
  if ((k_dtype == DSA_FP8_E4M3 || k_dtype == DSA_MXFP8_E4M3) && !k_scale) return DSA_ERR_NULL;
  if (q_dtype != DSA_F32 && q_dtype != DSA_BF16) return DSA_ERR_DTYPE;
  if (k_dtype != DSA_F32 && k_dtype != DSA_BF16 && k_dtype != DSA_FP8_E4M3 &&
      k_dtype != DSA_MXFP8_E4M3)
    return DSA_ERR_DTYPE;
  if (k_dtype == DSA_MXFP8_E4M3 && head_dim % 32 != 0) return DSA_ERR_SHAPE;
  if (n_heads < 1 || head_dim < 8 || head_dim % 8 != 0) return DSA_ERR_SHAPE;
  if ((int64_t)n_heads * head_dim > kGenericMaxHD || n_heads > kGenericMaxHeads)
    return DSA_ERR_UNSUPPORTED;
  if (top_k < 1) return DSA_ERR_SHAPE;
  if (top_k > DSA_MAX_TOPK) return DSA_ERR_UNSUPPORTED;
  dsa_status st = check_layout(layout, queries, true);
  if (st != DSA_OK) return st;
  if (misaligned(q) || misaligned(head_w) || misaligned(k_pool) || misaligned(k_scale) ||
      misaligned(out_idx) || misaligned(out_score) || misaligned(workspace))
    return DSA_ERR_ALIGN;
  const int32_t T = queries->num_queries;
  const IndexerPlan pl = plan_indexer(T, queries->max_visible, top_k, queries->total_visible);
  if (!workspace || workspace_bytes < pl.bytes) return DSA_ERR_WORKSPACE;

  IndexerParams p{};
  p.q = q;
  p.w = head_w;
  p.k_pool = k_pool;
  p.k_scale = (k_dtype == DSA_FP8_E4M3 || k_dtype == DSA_MXFP8_E4M3) ? k_scale : nullptr;
  p.L = make_layout(layout);
  p.q_seq = queries->q_seq;
  p.q_vis = queries->q_visible;
  p.T = T;
  p.H = n_heads;
  p.D = head_dim;
  p.K = top_k;
  p.max_visible = queries->max_visible;
  p.q_dtype = q_dtype;
  p.k_dtype = k_dtype;
  p.grid = pl.grid;
  p.split = pl.split;
  p.nsplit_max = pl.nsplit_max;
  p.cap = pl.cap;
  p.rs = pl.rs;
  p.compact = pl.compact;
  p.out_idx = out_idx;
  p.out_score = out_score;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  p.counters = reinterpret_cast<uint32_t*>(ws + pl.off_counters);
  p.hdr = reinterpret_cast<uint32_t*>(ws + pl.off_hdr);
  p.cand_key = reinterpret_cast<uint32_t*>(ws + pl.off_ckey);
  p.cand_pos = reinterpret_cast<int32_t*>(ws + pl.off_cpos);
  p.q_mx = reinterpret_cast<uint16_t*>(ws + pl.off_qmx);
  p.tl = timeline_buffer();
  const hipError_t e = launch_indexer(p, indexer_fast(q_dtype, k_dtype, n_heads, head_dim, layout),
                                      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DSA_OK : DSA_ERR_HIP;
}

size_t dsa_sparse_attn_workspace_size(int32_t num_queries, int32_t n_heads, int32_t top_k,
                                      int32_t d_v) {
  if (num_queries < 1 || n_heads < 1 || top_k < 1 || d_v < 1) return 0;
  // sized for the fast path, which needs at least as much as the reference path
  // the larger of the bf16-row and fp8-row plans (they may split the index list differently)
  const size_t a = plan_sfa(num_queries, n_heads, top_k, d_v, n_heads % 32 == 0, false).bytes;
  const size_t b = plan_sfa(num_queries, n_heads, top_k, d_v, n_heads % 32 == 0, true).bytes;
  return a > b ? a : b;
}

dsa_status dsa_sparse_attn(const void* q, dsa_dtype dtype, const void* kv_pool,
                           dsa_dtype kv_dtype, int32_t n_heads, int32_t d_qk, int32_t d_v,
                           float softmax_scale,
                           const dsa_layout* layout, const dsa_queries* queries,
                           const int32_t* idx, int32_t top_k, void* out, float* out_lse,
                           void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !kv_pool || !idx || !out) return DSA_ERR_NULL;
  if (dtype != DSA_F32 && dtype != DSA_BF16) return DSA_ERR_DTYPE;
  if (kv_dtype != dtype && !(kv_dtype == DSA_FP8_E4M3 && dtype == DSA_BF16)) return DSA_ERR_DTYPE;
  if (n_heads < 1 || n_heads > 1024) return DSA_ERR_SHAPE;
  if (kv_dtype == DSA_FP8_E4M3 && (d_qk != kSfaDqk || d_v != kSfaDv)) return DSA_ERR_UNSUPPORTED;
  if (d_qk < 64 || d_qk % 64 != 0 || d_v < 64 || d_v % 64 != 0 || d_v > d_qk) return DSA_ERR_SHAPE;
  if (d_qk > 1024) return DSA_ERR_UNSUPPORTED;
  if (top_k < 1) return DSA_ERR_SHAPE;
  if (top_k > DSA_MAX_TOPK) return DSA_ERR_UNSUPPORTED;
  if (!(softmax_scale == softmax_scale)) return DSA_ERR_SHAPE;
  dsa_status st = check_layout(layout, queries, false);
  if (st != DSA_OK) return st;
  if (misaligned(q) || misaligned(kv_pool) || misaligned(idx) || misaligned(out) ||
      misaligned(out_lse) || misaligned(workspace))
    return DSA_ERR_ALIGN;
  const int32_t T = queries->num_queries;
  const bool fast = sfa_fast(dtype, n_heads, d_qk, d_v);
  const SfaPlan pl = plan_sfa(T, n_heads, top_k, d_v, fast, kv_dtype == DSA_FP8_E4M3);
  if (!workspace || workspace_bytes < pl.bytes) return DSA_ERR_WORKSPACE;

  SfaParams p{};
  p.q = q;
  p.kv = kv_pool;
  p.L = make_layout(layout);
  p.q_seq = queries->q_seq;
  p.idx = idx;
  p.T = T;
  p.H = n_heads;
  p.dqk = d_qk;
  p.dv = d_v;
  p.K = top_k;
  p.scale = softmax_scale;
  p.dtype = dtype;
  p.kv_dtype = kv_dtype;
  p.heads_per_wg = pl.heads_per_wg;
  p.decode64 = pl.decode64;
  p.dim_waves = pl.dim_waves;
  p.n_hg = pl.n_hg;
  p.rows_per_split = pl.rows_per_split;
  p.nsplit = pl.nsplit;
  p.out = out;
  p.lse = out_lse;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  p.zero = ws + pl.off_zero;
  p.flags = reinterpret_cast<uint32_t*>(ws + pl.off_flags);
  p.part_o = ws + pl.off_part;
  p.part_ml = reinterpret_cast<float*>(ws + pl.off_ml);
  p.tl = timeline_buffer();
  const hipError_t e = launch_sfa(p, fast, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DSA_OK : DSA_ERR_HIP;
}

dsa_status dsa_store_index_keys(const float* k_new, int32_t n_tokens, int32_t head_dim,
                                const int64_t* slot, void* k_pool, dsa_dtype k_dtype,
                                float* k_scale, void* stream) {
  if (!k_new || !slot || !k_pool) return DSA_ERR_NULL;
  if ((k_dtype == DSA_FP8_E4M3 || k_dtype == DSA_MXFP8_E4M3) && !k_scale) return DSA_ERR_NULL;
  if (k_dtype != DSA_F32 && k_dtype != DSA_BF16 && k_dtype != DSA_FP8_E4M3 &&
      k_dtype != DSA_MXFP8_E4M3)
    return DSA_ERR_DTYPE;
  if (k_dtype == DSA_MXFP8_E4M3 && head_dim % 32 != 0) return DSA_ERR_SHAPE;
  if (n_tokens < 1 || n_tokens > (1 << 30) || head_dim < 1) return DSA_ERR_SHAPE;
  if (misaligned(k_new) || misaligned(slot) || misaligned(k_pool) || misaligned(k_scale))
    return DSA_ERR_ALIGN;
  const hipError_t e = launch_store_index_keys(k_new, n_tokens, head_dim, slot, k_pool, k_dtype,
                                               k_scale, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DSA_OK : DSA_ERR_HIP;
}

dsa_status dsa_store_kv(const void* kv_new, dsa_dtype src_dtype, int32_t n_tokens, int32_t d_qk,
                        const int64_t* slot, void* kv_pool, dsa_dtype pool_dtype, void* stream) {
  if (!kv_new || !slot || !kv_pool) return DSA_ERR_NULL;
  if ((src_dtype != DSA_F32 && src_dtype != DSA_BF16) ||
      (pool_dtype != DSA_F32 && pool_dtype != DSA_BF16 && pool_dtype != DSA_FP8_E4M3))
    return DSA_ERR_DTYPE;
  if (n_tokens < 1 || n_tokens > (1 << 30) || d_qk < 1) return DSA_ERR_SHAPE;
  if (pool_dtype == DSA_FP8_E4M3 && d_qk != kSfaDqk) return DSA_ERR_UNSUPPORTED;
  if (misaligned(kv_new) || misaligned(slot) || misaligned(kv_pool)) return DSA_ERR_ALIGN;
  const hipError_t e = launch_store_kv(kv_new, src_dtype, n_tokens, d_qk, slot, kv_pool,
                                       pool_dtype, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DSA_OK : DSA_ERR_HIP;
}

const char* dsa_status_string(dsa_status s) {
  switch (s) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_NULL: return "DSA_ERR_NULL: a required pointer is NULL";
    case DSA_ERR_SHAPE: return "DSA_ERR_SHAPE: a size is out of range or inconsistent";
    case DSA_ERR_DTYPE: return "DSA_ERR_DTYPE: dtype not accepted for this argument";
    case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED: shape or size not built";
    case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE: workspace missing or too small";
    case DSA_ERR_ALIGN: return "DSA_ERR_ALIGN: device pointer not 16-byte aligned";
    case DSA_ERR_HIP: return "DSA_ERR_HIP: HIP runtime or launch failure";
    case DSA_ERR_BLAS: return "DSA_ERR_BLAS: the library GEMM failed";
  }
  return "DSA_ERR_UNKNOWN";
}

int32_t dsa_abi_version(void) { return DSA_ABI_VERSION; }

size_t dsa_indexer_prolog_workspace_size(int32_t n_tokens, int32_t n_heads, int32_t head_dim) {
  if (n_tokens < 1 || n_heads < 1 || head_dim < 1) return 0;
  const int64_t N = (int64_t)n_heads * head_dim + head_dim + n_heads;
  return (size_t)((n_tokens * N * 4 + 255) / 256 * 256);
}

dsa_status dsa_indexer_prolog(const void* x, int32_t n_tokens, int32_t d_x, const void* w_proj,
                              const float* k_gain, float eps, int32_t n_heads, int32_t head_dim,
                              void* q_out, float* w_out, float* k_out, const int64_t* slot,
                              void* k_pool, dsa_dtype k_dtype, void* k_scale, void* workspace,
                              size_t workspace_bytes, void* stream) {
  if (!x || !w_proj || !k_gain || !q_out || !w_out) return DSA_ERR_NULL;
  if (!slot != !k_pool) return DSA_ERR_NULL;
  if (k_dtype != DSA_F32 && k_dtype != DSA_BF16 && k_dtype != DSA_FP8_E4M3 &&
      k_dtype != DSA_MXFP8_E4M3)
    return DSA_ERR_DTYPE;
  if (k_pool && (k_dtype == DSA_FP8_E4M3 || k_dtype == DSA_MXFP8_E4M3) && !k_scale)
    return DSA_ERR_NULL;
  if (n_tokens < 1 || n_tokens > (1 << 20) || d_x < 1 || n_heads < 1 || head_dim < 1 ||
      !(eps >= 0.f) || eps == INFINITY)
    return DSA_ERR_SHAPE;
  if (k_dtype == DSA_MXFP8_E4M3 && head_dim % 32 != 0) return DSA_ERR_SHAPE;
  const int64_t N = (int64_t)n_heads * head_dim + head_dim + n_heads;
  if (N > (1 << 30)) return DSA_ERR_SHAPE;
  if (head_dim > kPrologMaxD || (int64_t)n_heads * head_dim > (int64_t)65534 * 2048)
    return DSA_ERR_UNSUPPORTED;   // the epilogue's grid takes 2048 query values a workgroup
  const size_t need = dsa_indexer_prolog_workspace_size(n_tokens, n_heads, head_dim);
  if (!workspace || workspace_bytes < need) return DSA_ERR_WORKSPACE;
  if (misaligned(x) || misaligned(w_proj) || misaligned(k_gain) || misaligned(q_out) ||
      misaligned(w_out) || misaligned(k_out) || misaligned(slot) || misaligned(k_pool) ||
      misaligned(k_scale) || misaligned(workspace))
    return DSA_ERR_ALIGN;
  PrologParams p{};
  p.y = static_cast<const float*>(workspace);
  p.N = (int32_t)N;
  p.H = n_heads;
  p.D = head_dim;
  p.eps = eps;
  p.gain = k_gain;
  p.q_out = q_out;
  p.q_mx = k_dtype == DSA_MXFP8_E4M3;
  p.w_out = w_out;
  p.k_out = k_out;
  p.slot = slot;
  p.pool = k_pool;
  p.k_dt = k_dtype;
  p.k_scale = static_cast<float*>(k_scale);
  int blas = 0;
  const hipError_t e = run_prolog(x, n_tokens, d_x, w_proj, p, static_cast<hipStream_t>(stream), &blas);
  if (blas) return DSA_ERR_BLAS;
  return e == hipSuccess ? DSA_OK : DSA_ERR_HIP;
}

dsa_status dsa_zigzag_ranges(int64_t n_tokens, int32_t n_shards, int32_t shard, int64_t* ranges) {
  if (!ranges) return DSA_ERR_NULL;
  if (n_tokens < 0 || n_shards < 1 || shard < 0 || shard >= n_shards) return DSA_ERR_SHAPE;
  // segment bounds floor(s * n / m) without overflow for n < 2^62: n = a * m + b
  const int64_t m = 2 * (int64_t)n_shards, a = n_tokens / m, b = n_tokens % m;
  auto bound = [&](int64_t s) { return s * a + s * b / m; };
  const int64_t tail = m - 1 - shard;
  ranges[0] = bound(shard);
  ranges[1] = bound(shard + 1);
  ranges[2] = bound(tail);
  ranges[3] = bound(tail + 1);
  return DSA_OK;
}

}  // extern "C"
