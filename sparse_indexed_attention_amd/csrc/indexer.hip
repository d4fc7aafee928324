// Lightning indexer fused with exact Top-K (gfx950).
//
// What it computes: for query t of sequence b, visible prefix V, and each position s < V,
//   S[s] = sum_h w[t,h] * ReLU(q[t,h,:] . key(s))
// then the K_eff = min(K, V) best positions (score descending, lower position first).
// Scoring, head-weighted aggregation and Top-K run in one kernel that reads the paged key
// cache directly and writes only the index list: the fused index operator of "Large Model
// Inference Acceleration: Day-0 Adaptation..." (section 1.1) and of "Day0 Adaptation and
// Sparse Attention Optimization for Long-Sequence LLM Inference" (section 4).  The
// per-head scores never leave the registers and the per-position scores stay in LDS.
//
// Work decomposition (MI355X: 256 CUs, wave64, 160 KB LDS per CU):
//   * one workgroup per (query, context split of `split` positions);
//   * scoring: each wave takes groups of 32 positions; one v_mfma_f32_32x32x16_bf16 chain
//     per 32-head half computes x[head, position] for the group (keys as the B operand,
//     straight from HBM in MFMA lane layout; fp8 keys are widened to bf16 exactly), then each
//     lane applies ReLU and the head weights to the 16 accumulator rows it holds and one
//     cross-lane add finishes the head sum.  The fp8 per-token scale multiplies the head sum
//     (ReLU(c x) = c ReLU(x) for c > 0).  Every position goes through the same instruction
//     sequence, so bit-identical keys get bit-identical scores wherever they sit;
//   * each split picks a threshold key with radix histograms over its LDS scores so that a
//     little more than its expected share of the Top-K survives, and writes those
//     candidates (order-preserving key, position) to the workspace;
//   * the last split of a query to arrive (atomic counter) gathers the candidates, finds the
//     exact K_eff-th key by radix select, and checks that every split's threshold lies at or
//     below it - then the candidates provably contain the exact answer.  A split whose
//     threshold was too high is re-scored by the merging workgroup and contributes its exact
//     local Top-K instead (rare for any input whose top positions are not concentrated in a
//     few splits; always correct).
// A query whose prefix fits one split does the exact selection in place.
// A reference path (any supported dtypes and head geometry) scores each position in fp64.

#include "dsa_internal.hpp"

namespace dsa {
namespace {

constexpr int NT = kIdxThreads;

struct Smem {
  uint32_t keys[kSplitMax];
  int hist[256];
  int res[4];
  int scan[NT / 64 + 2];
  int seg_off[kNSplitMax + 1];
  uint32_t seg_tau[kNSplitMax];
  int bcast[4];
};

struct GenericSmem {
  float q[kGenericMaxHD];
  float w[kGenericMaxHeads];
};

// ---------------------------------------------------------------------------------------
// Scoring
// ---------------------------------------------------------------------------------------

// MFMA scorer: q bf16 [64 heads x 128 dims], keys bf16 or fp8 (128 per token).
// Lane layout of v_mfma_f32_32x32x16_bf16: lane l supplies row/column (l & 31) and the
// 8-element k-slice 8*(l >> 5) .. +7; accumulator element r of lane l is
// D[8*(r/4) + 4*(l>>5) + (r%4)][l & 31].  The 128 key dims are assigned to k-slices so that
// lane half h reads dims [64h, 64h+64) of its key row contiguously; the query uses the same
// assignment, so every MFMA step still pairs equal dims.
template <bool FP8>
__device__ __forceinline__ void score_mfma(const IndexerParams& p, int t, int seq, int start,
                                           int len, uint32_t* lkeys) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, col = lane & 31;
  const uint16_t* qb = (const uint16_t*)p.q + (size_t)t * (64 * 128);
  bf16x8 a0[8], a1[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    a0[s] = *(const bf16x8*)(qb + col * 128 + half * 64 + 8 * s);
    a1[s] = *(const bf16x8*)(qb + (32 + col) * 128 + half * 64 + 8 * s);
  }
  float w0[16], w1[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = 8 * (r >> 2) + 4 * half + (r & 3);
    w0[r] = p.w[t * 64 + i];
    w1[r] = p.w[t * 64 + 32 + i];
  }
  constexpr int NV = FP8 ? 4 : 8;             // 16-byte loads per lane per group
  constexpr int ROWB = FP8 ? 128 : 256;       // bytes per key row
  const uint8_t* kbase = (const uint8_t*)p.k_pool + half * (ROWB / 2);
  const int ngroups = (len + 31) >> 5;

  auto load = [&](int g, u32x4* raw, float& sc) {
    const int off = g * 32 + col;
    if (off < len) {
      const int64_t row = pool_row(p.L, seq, start + off);
      const u32x4* src = (const u32x4*)(kbase + row * ROWB);
#pragma unroll
      for (int i = 0; i < NV; ++i) raw[i] = __builtin_nontemporal_load(src + i);
      sc = FP8 ? p.k_scale[row] : 1.f;
    } else {
#pragma unroll
      for (int i = 0; i < NV; ++i) raw[i] = u32x4{0u, 0u, 0u, 0u};
      sc = 0.f;
    }
  };

  u32x4 cur[NV], nxt[NV];
  float csc = 0.f, nsc = 0.f;
  int g = wave;
  if (g < ngroups) load(g, cur, csc);
  for (; g < ngroups; g += 4) {
    const bool more = g + 4 < ngroups;
    if (more) load(g + 4, nxt, nsc);
    f32x16 acc0 = {}, acc1 = {};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      bf16x8 b;
      if constexpr (FP8) {
        const u32x4 v = cur[s >> 1];
        const uint32_t lo = (s & 1) ? v.z : v.x;
        const uint32_t hi = (s & 1) ? v.w : v.y;
        const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
        const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
        const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
        const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
        b = bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
      } else {
        b = __builtin_bit_cast(bf16x8, cur[s]);
      }
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[s], b, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[s], b, acc1, 0, 0, 0);
    }
    float part = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) part = fmaf(w0[r], fmaxf(acc0[r], 0.f), part);
#pragma unroll
    for (int r = 0; r < 16; ++r) part = fmaf(w1[r], fmaxf(acc1[r], 0.f), part);
    float tot = part + __shfl_xor(part, 32, 64);
    if constexpr (FP8) tot *= csc;
    const int off = g * 32 + col;
    if (half == 0 && off < len) lkeys[off] = float_to_key(tot);
    if (more) {
#pragma unroll
      for (int i = 0; i < NV; ++i) cur[i] = nxt[i];
      csc = nsc;
    }
  }
}

__device__ __forceinline__ float load_elem(const void* base, int dt, int64_t i) {
  if (dt == kDtF32) return ((const float*)base)[i];
  if (dt == kDtBF16) return bf16_bits_to_f32(((const uint16_t*)base)[i]);
  return fp8_e4m3_to_f32(((const uint8_t*)base)[i]);
}

// Reference scorer: one thread per position, fp64 accumulation (products of the stored
// operands are exact in fp64), rounded once to fp32.
__device__ void score_generic(const IndexerParams& p, int seq, int start, int len,
                              uint32_t* lkeys, const GenericSmem& gs) {
  const int H = p.H, D = p.D;
  for (int i = threadIdx.x; i < len; i += NT) {
    const int64_t row = pool_row(p.L, seq, start + i);
    const double ks = (p.k_dtype == kDtFP8) ? (double)p.k_scale[row] : 1.0;
    double S = 0.0;
    for (int h = 0; h < H; ++h) {
      double x = 0.0;
      for (int d = 0; d < D; ++d)
        x = fma((double)gs.q[h * D + d], (double)load_elem(p.k_pool, p.k_dtype, row * D + d) * ks, x);
      S = fma((double)gs.w[h], fmax(x, 0.0), S);
    }
    lkeys[i] = float_to_key((float)S);
  }
}

template <int MODE>
__device__ __forceinline__ void score_split(const IndexerParams& p, int t, int seq, int start,
                                            int len, uint32_t* lkeys, const GenericSmem* gs) {
  if constexpr (MODE == 1) score_mfma<false>(p, t, seq, start, len, lkeys);
  else if constexpr (MODE == 2) score_mfma<true>(p, t, seq, start, len, lkeys);
  else score_generic(p, seq, start, len, lkeys, *gs);
}

// ---------------------------------------------------------------------------------------
// Radix selection over order-preserving keys
// ---------------------------------------------------------------------------------------

// Histogram of digit (key >> shift) & 255 over keys with (key & mask) == prefix.  The first
// digit of a set of scores is nearly constant, so that pass aggregates equal digits across
// the wave before touching LDS (one atomic per distinct digit instead of 64 on one word).
template <class Get>
__device__ void build_hist(Get get, int n, uint32_t prefix, uint32_t mask, int shift, int* hist,
                           bool aggregate) {
  for (int i = threadIdx.x; i < 256; i += NT) hist[i] = 0;
  __syncthreads();
  if (aggregate) {
    const int lane = threadIdx.x & 63;
    const int iters = (n + NT - 1) / NT;
    for (int it = 0; it < iters; ++it) {
      const int i = it * NT + threadIdx.x;
      bool m = false;
      int bin = 0;
      if (i < n) {
        const uint32_t k = get(i);
        m = (k & mask) == prefix;
        bin = (int)((k >> shift) & 255u);
      }
      uint64_t todo = __ballot(m);
      while (todo) {
        const int leader = __builtin_ctzll(todo);
        const int lb = __shfl(bin, leader, 64);
        const uint64_t grp = __ballot(m && bin == lb) & todo;
        if (lane == leader) atomicAdd(&hist[lb], __popcll(grp));
        todo &= ~grp;
      }
    }
  } else {
    for (int i = threadIdx.x; i < n; i += NT) {
      const uint32_t k = get(i);
      if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1);
    }
  }
  __syncthreads();
}

// Bin d holding the r-th largest (1-based) counted key: above(d) < r <= above(d) + hist[d],
// above(d) = number of counted keys in bins > d.  res = {d, above(d), hist[d]}.
__device__ void radix_find(const int* hist, int r, int* res) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int c[4], loc = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      c[u] = hist[255 - 4 * lane - u];
      loc += c[u];
    }
    int above = wave_inclusive_scan(loc) - loc;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (above < r && r <= above + c[u]) {
        res[0] = 255 - 4 * lane - u;
        res[1] = above;
        res[2] = c[u];
      }
      above += c[u];
    }
  }
  __syncthreads();
}

// The k-th largest key (1 <= k <= n) and the number of keys strictly above it.
template <class Get>
__device__ void radix_kth(Get get, int n, int k, Smem& sm, uint32_t& T, int& gt) {
  uint32_t prefix = 0, mask = 0;
  int above = 0;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    build_hist(get, n, prefix, mask, shift, sm.hist, pass == 0);
    radix_find(sm.hist, k - above, sm.res);
    const int d = sm.res[0], a = sm.res[1];
    above += a;
    prefix |= (uint32_t)d << shift;
    mask |= 0xffu << shift;
  }
  T = prefix;
  gt = above;
}

// A threshold key tau such that the count of keys >= tau is at least m when possible and
// at most `hard`, preferably at most `soft`.  Returns tau and that count.
__device__ void local_threshold(const uint32_t* keys, int n, int m, int soft, int hard, Smem& sm,
                                uint32_t& tau, int& count) {
  auto get = [&](int i) { return keys[i]; };
  uint32_t prefix = 0, mask = 0;
  int above = 0;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    build_hist(get, n, prefix, mask, shift, sm.hist, pass == 0);
    radix_find(sm.hist, m - above, sm.res);
    const int d = sm.res[0], a = sm.res[1], c = sm.res[2];
    const int tot = above + a + c;
    const uint32_t edge = prefix | ((uint32_t)d << shift);
    if (tot <= soft || (pass == 3 && tot <= hard)) {
      tau = edge;
      count = tot;
      return;
    }
    above += a;
    prefix = edge;
    mask |= 0xffu << shift;
  }
  // One value v = prefix holds too many equal keys: keep only the keys above it.
  tau = prefix + 1u;
  count = above;
}

// Stable selection in index order: element i is taken if key > T, or key == T and fewer than
// `need` earlier elements equal to T were taken.  out(slot, i, key) for each taken element.
template <class Get, class Out>
__device__ void emit(Get get, int n, uint32_t T, int need, Out out, Smem& sm) {
  const int E = (n + NT - 1) / NT;
  const int lo = min(n, (int)threadIdx.x * E), hi = min(n, lo + E);
  int eq = 0;
  for (int i = lo; i < hi; ++i) eq += get(i) == T;
  int tot;
  const int eq_base = wg_exclusive_scan<NT>(eq, sm.scan, &tot);
  int sel = 0, r = eq_base;
  for (int i = lo; i < hi; ++i) {
    const uint32_t k = get(i);
    if (k > T) ++sel;
    else if (k == T) { sel += r < need; ++r; }
  }
  int slot = wg_exclusive_scan<NT>(sel, sm.scan, &tot);
  r = eq_base;
  for (int i = lo; i < hi; ++i) {
    const uint32_t k = get(i);
    bool take = false;
    if (k > T) take = true;
    else if (k == T) { take = r < need; ++r; }
    if (take) out(slot++, i, k);
  }
}

__device__ void pad_output(const IndexerParams& p, int t, int from) {
  for (int s = from + (int)threadIdx.x; s < p.K; s += NT) {
    p.out_idx[(size_t)t * p.K + s] = -1;
    if (p.out_score) p.out_score[(size_t)t * p.K + s] = 0.f;
  }
}

// Exact local Top-kk of the split scores in LDS, written to the candidate slots of split j.
__device__ void split_exact_candidates(const IndexerParams& p, int t, int j, int start, int len,
                                       int kk, Smem& sm) {
  auto lget = [&](int i) { return sm.keys[i]; };
  uint32_t T;
  int gt;
  radix_kth(lget, len, kk, sm, T, gt);
  const size_t cb = ((size_t)t * p.nsplit_max + j) * p.cap;
  emit(lget, len, T, kk - gt,
       [&](int slot, int i, uint32_t k) {
         p.cand_key[cb + slot] = k;
         p.cand_pos[cb + slot] = start + i;
       },
       sm);
}

// ---------------------------------------------------------------------------------------
// Kernel
// ---------------------------------------------------------------------------------------
template <int MODE>
__global__ __launch_bounds__(NT) void indexer_topk_kernel(IndexerParams p) {
  __shared__ Smem sm;
  const int t = blockIdx.y, j = blockIdx.x;
  const int V = min(p.q_vis[t], p.max_visible);
  if (V <= 0) {
    if (j == 0) pad_output(p, t, 0);
    return;
  }
  const int nsplit = (V + p.split - 1) / p.split;
  if (j >= nsplit) return;
  const int seq = p.q_seq[t];
  const int K_eff = min(p.K, V);
  const int start = j * p.split, len = min(p.split, V - start);

  const GenericSmem* gsp = nullptr;
  if constexpr (MODE == 0) {
    __shared__ GenericSmem gs;
    const int HD = p.H * p.D;
    for (int i = threadIdx.x; i < HD; i += NT)
      gs.q[i] = load_elem(p.q, p.q_dtype, (int64_t)t * HD + i);
    for (int i = threadIdx.x; i < p.H; i += NT) gs.w[i] = p.w[(size_t)t * p.H + i];
    __syncthreads();
    gsp = &gs;
  }

  score_split<MODE>(p, t, seq, start, len, sm.keys, gsp);
  __syncthreads();
  auto lget = [&](int i) { return sm.keys[i]; };

  if (nsplit == 1) {
    uint32_t T;
    int gt;
    radix_kth(lget, len, K_eff, sm, T, gt);
    emit(lget, len, T, K_eff - gt,
         [&](int slot, int i, uint32_t k) {
           p.out_idx[(size_t)t * p.K + slot] = start + i;
           if (p.out_score) p.out_score[(size_t)t * p.K + slot] = key_to_float(k);
         },
         sm);
    pad_output(p, t, K_eff);
    return;
  }

  // ---- candidates of this split --------------------------------------------------------
  {
    const float e = (float)K_eff * (float)len / (float)V;
    int m = (int)ceilf(e + 4.f * sqrtf(e) + 4.f);
    const int hard = min(len, p.cap);
    m = min(m, hard);
    const int soft = min(hard, 2 * m);
    uint32_t tau = 0u;
    int cnt = len;
    if (m < len) local_threshold(sm.keys, len, m, soft, hard, sm, tau, cnt);
    else tau = 0u;       // everything fits: all keys are >= 0
    const size_t cb = ((size_t)t * p.nsplit_max + j) * p.cap;
    emit(lget, len, tau, 0x7fffffff,
         [&](int slot, int i, uint32_t k) {
           if (slot < p.cap) {
             p.cand_key[cb + slot] = k;
             p.cand_pos[cb + slot] = start + i;
           }
         },
         sm);
    if (threadIdx.x == 0) {
      uint32_t* h = p.hdr + ((size_t)t * p.nsplit_max + j) * 2;
      h[0] = (uint32_t)min(cnt, p.cap);
      h[1] = tau;
    }
  }

  // ---- arrival: the last split of this query merges --------------------------------------
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0)
    sm.bcast[0] = atomicAdd(&p.counters[t], 1u) == (uint32_t)(nsplit - 1);
  __syncthreads();
  if (!sm.bcast[0]) return;
  __threadfence();

  const uint32_t* hdr = p.hdr + (size_t)t * p.nsplit_max * 2;
  const size_t qbase = (size_t)t * p.nsplit_max * p.cap;
  uint32_t* fk = p.flat_key + qbase;
  int32_t* fpos = p.flat_pos + qbase;

  for (int round = 0; round < 2; ++round) {
    // split headers -> LDS, candidate offsets
    int c[4], loc = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int jj = threadIdx.x * 4 + u;
      c[u] = 0;
      if (jj < nsplit) {
        c[u] = (int)__builtin_nontemporal_load(hdr + 2 * jj);
        sm.seg_tau[jj] = __builtin_nontemporal_load(hdr + 2 * jj + 1);
      }
      loc += c[u];
    }
    int N;
    int base = wg_exclusive_scan<NT>(loc, sm.scan, &N);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int jj = threadIdx.x * 4 + u;
      if (jj < nsplit) sm.seg_off[jj] = base;
      base += c[u];
    }
    if (threadIdx.x == 0) sm.seg_off[nsplit] = N;
    __syncthreads();

    // gather the candidates into one flat array (split order = position order)
    {
      const int E = (N + NT - 1) / NT;
      const int lo = min(N, (int)threadIdx.x * E), hi = min(N, lo + E);
      if (lo < hi) {
        int a = 0, b = nsplit - 1;      // last split with seg_off <= lo
        while (a < b) {
          const int mid = (a + b + 1) >> 1;
          if (sm.seg_off[mid] <= lo) a = mid; else b = mid - 1;
        }
        int jj = a;
        for (int i = lo; i < hi; ++i) {
          while (i >= sm.seg_off[jj + 1]) ++jj;
          const size_t src = qbase + (size_t)jj * p.cap + (i - sm.seg_off[jj]);
          fk[i] = __builtin_nontemporal_load(p.cand_key + src);
          fpos[i] = __builtin_nontemporal_load(p.cand_pos + src);
        }
      }
    }
    __threadfence();
    __syncthreads();

    auto fget = [&](int i) { return __builtin_nontemporal_load(fk + i); };
    const bool enough = N >= K_eff;
    uint32_t T = 0u;
    int gt = 0;
    if (enough) radix_kth(fget, N, K_eff, sm, T, gt);
    int bad = 0;
    for (int jj = threadIdx.x; jj < nsplit; jj += NT)
      bad |= enough ? (sm.seg_tau[jj] > T) : (sm.seg_tau[jj] != 0u);
    bad = __syncthreads_or(bad);

    if (!bad || round == 1) {
      emit(fget, N, T, K_eff - gt,
           [&](int slot, int i, uint32_t k) {
             if (slot < K_eff) {
               p.out_idx[(size_t)t * p.K + slot] = __builtin_nontemporal_load(fpos + i);
               if (p.out_score) p.out_score[(size_t)t * p.K + slot] = key_to_float(k);
             }
           },
           sm);
      pad_output(p, t, K_eff);
      if (threadIdx.x == 0) p.counters[t] = 0u;
      return;
    }

    // Fallback: splits whose threshold cut above the K_eff-th key contribute their exact
    // local Top-K instead.
    for (int jj = 0; jj < nsplit; ++jj) {
      const bool fail = enough ? (sm.seg_tau[jj] > T) : (sm.seg_tau[jj] != 0u);
      if (!fail) continue;
      const int s0 = jj * p.split, l0 = min(p.split, V - s0);
      __syncthreads();
      score_split<MODE>(p, t, seq, s0, l0, sm.keys, gsp);
      __syncthreads();
      const int kk = min(l0, K_eff);
      split_exact_candidates(p, t, jj, s0, l0, kk, sm);
      if (threadIdx.x == 0) {
        uint32_t* h = p.hdr + ((size_t)t * p.nsplit_max + jj) * 2;
        h[0] = (uint32_t)kk;
        h[1] = 0u;
      }
    }
    __threadfence();
    __syncthreads();
  }
}

}  // namespace

IndexerPlan plan_indexer(int32_t T, int32_t max_visible, int32_t top_k) {
  IndexerPlan pl{};
  const int64_t target_wg = 1024;
  int64_t split = ((int64_t)T * max_visible + target_wg - 1) / target_wg;
  split = (split + 63) / 64 * 64;
  if (split < 512) split = 512;
  if (split > kSplitMax) split = kSplitMax;
  // long prefixes need larger splits to stay within kNSplitMax
  while ((max_visible + split - 1) / split > kNSplitMax && split < kSplitMax) split += 64;
  pl.split = (int32_t)split;
  pl.nsplit_max = (int32_t)((max_visible + split - 1) / split);
  pl.cap = (int32_t)(split < top_k ? split : top_k);
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t slots = (size_t)T * pl.nsplit_max * pl.cap;
  size_t off = 0;
  pl.off_counters = off; off = al(off + (size_t)T * 4);
  pl.off_hdr = off;      off = al(off + (size_t)T * pl.nsplit_max * 8);
  pl.off_ckey = off;     off = al(off + slots * 4);
  pl.off_cpos = off;     off = al(off + slots * 4);
  pl.off_fkey = off;     off = al(off + slots * 4);
  pl.off_fpos = off;     off = al(off + slots * 4);
  pl.bytes = off;
  return pl;
}

hipError_t launch_indexer(const IndexerParams& p, bool fast_path, hipStream_t stream) {
  const dim3 grid(p.nsplit_max, p.T), block(NT);
  if (!fast_path) hipLaunchKernelGGL(indexer_topk_kernel<0>, grid, block, 0, stream, p);
  else if (p.k_dtype == kDtFP8) hipLaunchKernelGGL(indexer_topk_kernel<2>, grid, block, 0, stream, p);
  else hipLaunchKernelGGL(indexer_topk_kernel<1>, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace dsa
