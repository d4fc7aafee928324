// Sparse Flash Attention over selected rows of the paged MLA latent cache (gfx950).
//
// For query t and head h:  z_j = scale * q[t,h,:] . R_j,  out[t,h,:] = softmax(z) . R[:, :d_v],
// where R_j is the 576-wide latent row of the j-th selected position and its first 512
// columns are the value.  SFA reads the main KV only at the indexer's positions ("Day0
// Adaptation and Performance Optimization for Novel Long-Sequence Reasoning Models",
// section 3); rows are fetched whole with 16-byte vector reads, the block-wise vectorized
// sparse reads of "Day0 Adaptation and Sparse Attention Optimization for Long-Sequence LLM
// Inference", section 4.
//
// Fast path (bf16 storage, d_qk = 576, d_v = 512, heads a multiple of 32): a workgroup owns
// (query, group of 32*NW heads, slice of the index list); every selected row is read once per
// workgroup and serves all of its heads.
//   * Gather: tiles of 32 rows land in LDS through direct-to-LDS loads, double-buffered (tile
//     i+1 streams in while tile i is computed).  LDS rows are 73 sixteen-byte chunks (one of
//     padding): with that odd stride both the MFMA reads of 16 rows at one column and the
//     transposing reads of 4 rows x 2 chunks touch distinct banks.  The pool rows of the slice
//     are resolved once, into LDS.
//   * Each wave holds 32 heads.  S^T = R . Q^T on v_mfma_f32_32x32x16_bf16: tile rows are the
//     A operand and the wave's queries (registers) the B operand, so a lane column is a head.
//   * Online softmax in the exp2 domain; the output accumulators are rescaled only when a
//     head's running maximum moves.
//   * O += P . V on the same MFMA: the probabilities, in the S^T accumulator layout, are the
//     A operand as they stand (the k order of the contraction is permuted to the rows each
//     lane holds), and the V operand comes straight from the row-major tile through the
//     transposing LDS read ds_read_b64_tr_b16, which gathers one dim of four rows into a lane.
//   * Slices of the index list are merged by a log-sum-exp weighted combine kernel.
// Reference path (fp32 storage or other shapes): one workgroup per (query, head), fp32.

#include <cstdlib>

#include "dsa_internal.hpp"

namespace dsa {
namespace {

constexpr int kTileRows = 32;
constexpr int kRowBytes = kSfaDqk * 2;                   // 1152
constexpr int kRowChunks = kRowBytes / 16;               // 72 sixteen-byte chunks per row
constexpr int kLdsChunks = kRowChunks + 1;               // LDS row stride, in chunks
constexpr int kTileSlots = kTileRows * kLdsChunks;       // 2336
constexpr int kTileBytes = kTileSlots * 16;              // 37376
constexpr int kTileLoads = (kTileSlots + 63) / 64;       // 37 direct-to-LDS loads per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Byte offset in a tile of chunk c of row r.
__device__ __forceinline__ int tile_off(int r, int c) { return 16 * (r * kLdsChunks + c); }

__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt((N & 0xf) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// 16 bytes per active lane from a per-lane global address into LDS at lds + 16 * lane (lds is
// wave-uniform).  Inline asm keeps the compiler's wait insertion from draining all loads
// before every LDS read; the caller waits with vmcnt.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void load16_to_lds(const void* gaddr, uint32_t lds_in) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_in);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(gaddr), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop

// Row of the 32x32 MFMA accumulator element r held by lane half h (lane column = l & 31).
__device__ __forceinline__ int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

template <int NW>
__global__ __launch_bounds__(NW * 64, 1) void sfa_mfma_kernel(SfaParams p) {
  constexpr int NTS = NW * 64;
  constexpr int LPW = (kTileLoads + NW - 1) / NW;  // loads per wave per tile (at most)
  constexpr int LPW_MIN = kTileLoads / NW;          // ... and at least
  __shared__ __attribute__((aligned(16))) uint8_t tiles[2][kTileBytes];
  __shared__ int32_t rows[kMaxTopK];                // pool row of each slice entry, -1 if none
  __shared__ __attribute__((aligned(16))) float hv[NW][32];   // per-head values of a wave

  // workgroup -> (query, head group, slice); consecutive workgroups go to different XCDs, so
  // the head groups of one (query, slice) are placed 8 apart and share an XCD's L2
  const int wg = blockIdx.x;
  const int xcd = wg & 7, qq = wg >> 3;
  const int hg = qq % p.n_hg;
  const int cc = (qq / p.n_hg) * 8 + xcd;
  if (cc >= p.T * p.nsplit) return;
  const int t = cc / p.nsplit, r = cc - t * p.nsplit;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5, c = lane & 31;          // lane half, lane column (= head)
  const int h0 = hg * p.heads_per_wg + wave * 32;
  const int seq = p.q_seq[t];
  const int j0 = r * p.rows_per_split;
  const int nrows = min(p.K, j0 + p.rows_per_split) - j0;
  const int ntiles = (nrows + kTileRows - 1) / kTileRows;

  // pool rows of the slice
  {
    const int32_t* idx = p.idx + (size_t)t * p.K + j0;
    for (int i = tid; i < ntiles * kTileRows; i += NTS) {
      const int pos = i < nrows ? idx[i] : -1;
      rows[i] = pos >= 0 ? (int32_t)pool_row(p.L, seq, pos) : -1;
    }
  }
  // queries of this wave's 32 heads: lane holds head c, dims 16s + 8hh .. +7
  bf16x8 qk[36];
  {
    const uint16_t* qb = (const uint16_t*)p.q + ((size_t)t * p.H + h0 + c) * kSfaDqk + 8 * hh;
#pragma unroll
    for (int s = 0; s < 36; ++s) qk[s] = *(const bf16x8*)(qb + 16 * s);
  }
  wait_vmcnt<0>();
  __syncthreads();

  const uint8_t* kv = (const uint8_t*)p.kv;
  // This wave's share of tile `tile`: loads I = wave, wave + NW, ...; lane l of load I fills
  // chunk slot 64 I + l.  Padding slots are skipped; rows without a position get zeros.
  auto issue = [&](int tile, int buf) {
    uint8_t* tb = tiles[buf];
#pragma unroll
    for (int u = 0; u < LPW; ++u) {
      const int I = wave + NW * u;
      if (LPW != LPW_MIN && I >= kTileLoads) break;
      const int P = 64 * I + lane;
      const int rr = P / kLdsChunks, ch = P - rr * kLdsChunks;
      if (P < kTileSlots && ch < kRowChunks) {
        const int row = rows[tile * kTileRows + rr];
        if (row >= 0) load16_to_lds(kv + (size_t)row * kRowBytes + 16 * ch, lds_u32(tb + 1024 * I));
        else *(u32x4*)(tb + 16 * P) = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };

  const float scale2 = p.scale * kLog2e;
  const int* rowsp = rows;

  // S^T = R . Q^T for the tile in `tb`, scaled to the exp2 domain, -inf for empty rows: lane
  // (hh, c) gets rows acc_row(e, hh) of head c.  Scheduling fences every few steps keep the
  // operand reads close to their MFMAs: the register file holds the queries and the output
  // accumulators, little else.
  auto scores = [&](const uint8_t* tb, int tile, float (&z)[16]) {
    f32x16 sa = {};
    const uint8_t* ra = tb + tile_off(c, hh);
#pragma unroll
    for (int s0 = 0; s0 < 36; s0 += 4) {
      bf16x8 a[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) a[u] = *(const bf16x8*)(ra + 32 * (s0 + u));
#pragma unroll
      for (int u = 0; u < 4; ++u) sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[u], qk[s0 + u], sa, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    const int* trow = rowsp + tile * kTileRows;
#pragma unroll
    for (int e = 0; e < 16; ++e) z[e] = trow[acc_row(e, hh)] >= 0 ? sa[e] * scale2 : -INFINITY;
  };
  // Double-buffered walk over the slice's tiles: body(tile, tb) runs once each tile is in LDS.
  auto walk = [&](auto body) {
    issue(0, 0);
    for (int tile = 0; tile < ntiles; ++tile) {
      const int buf = tile & 1;
      if (tile + 1 < ntiles) {
        issue(tile + 1, buf ^ 1);
        wait_vmcnt<LPW_MIN>();                    // this wave's loads of `tile` have landed
      } else {
        wait_vmcnt<0>();
      }
      __syncthreads();                            // ... and every other wave's
      body(tile, tiles[buf]);
      __syncthreads();                            // the buffer is refilled two tiles later
    }
  };

  // Exponent reference m2 per head: set by the head's first live tile and never moved, so the
  // output accumulators are never rescaled.  Probabilities exp2(z - m2) may exceed 1; up to
  // 2^64 bf16 operands and fp32 sums of 2^11 terms keep their full relative precision.  A
  // head whose scores pass m2 + 64 is flagged, and the combine kernel recomputes it with the
  // reference method.
  float m2 = -INFINITY, l = 0.f;
  f32x16 o[16];
  bool over = false;
  auto attend = [&](int tile, const uint8_t* tb) {
    float z[16];
    scores(tb, tile, z);
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = fmaxf(mx, z[e]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    if (m2 == -INFINITY) m2 = mx;                // first live tile of this head (O, l are 0)
    over |= mx > m2 + 64.f;
    const bool live = m2 != -INFINITY;
    float pe[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      pe[e] = live ? exp2f(z[e] - m2) : 0.f;
      l += pe[e];
    }
    // P as the A operand of k step kk: k slot 8hh + u is row 16kk + 8(u/4) + 4hh + u%4,
    // i.e. accumulator elements 8kk .. 8kk+7 as they stand
    bf16x8 pa0, pa1;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      pa0[u] = (__bf16)pe[u];
      pa1[u] = (__bf16)pe[8 + u];
    }
    // V operand for dims 32nb .. +31, k step kk: in each 16-lane group, lane i supplies row
    // 16kk + 8jj + 4hh + i/4, dims 32nb + 16(c/16) + 4(i%4) .. +3; the transposing read
    // returns dim 32nb + c of four consecutive rows
    const int vi = c & 15;
    const int vrow = 4 * hh + (vi >> 2);
    const int vdim = 16 * (c >> 4) + 4 * (vi & 3);
#pragma unroll
    for (int nb = 0; nb < 16; ++nb) {
      const int dim = 32 * nb + vdim;
      const int cho = tile_off(0, dim >> 3) + 2 * (dim & 7);
      bf16x8 b[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(tb + tile_off(16 * kk + vrow, 0) + cho));
        const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(tb + tile_off(16 * kk + 8 + vrow, 0) + cho));
        b[kk] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
      }
      o[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa0, b[0], o[nb], 0, 0, 0);
      o[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa1, b[1], o[nb], 0, 0, 0);
      if (nb & 1) __builtin_amdgcn_sched_barrier(0);
    }
  };

#pragma unroll
  for (int n = 0; n < 16; ++n) o[n] = f32x16{};
  walk(attend);
  if (over && hh == 0) p.flags[(size_t)t * p.H + h0 + c] = 1u;

  // per-head totals: the two lane halves of a column hold disjoint rows of its head
  const float lt = l + __shfl_xor(l, 32, 64);
  if (p.nsplit == 1) {
    if (hh == 0) hv[wave][c] = lt > 0.f ? 1.f / lt : 0.f;
    uint16_t* out = (uint16_t*)p.out + ((size_t)t * p.H + h0) * kSfaDv;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 inv = *(const f32x4*)&hv[wave][8 * j + 4 * hh];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hd = 8 * j + 4 * hh + i;
#pragma unroll
        for (int nb = 0; nb < 16; ++nb)
          out[hd * kSfaDv + 32 * nb + c] = __builtin_bit_cast(uint16_t, (__bf16)(o[nb][4 * j + i] * inv[i]));
      }
    }
    if (p.lse && hh == 0)
      p.lse[(size_t)t * p.H + h0 + c] = lt > 0.f ? (m2 + log2f(lt)) * kLn2 : -INFINITY;
  } else {
    // partial (unnormalised O, running max in the exp2 domain, sum) of this slice
    const size_t pb = (((size_t)t * p.H + h0) * p.nsplit + r);   // (t, head h0, slice r)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hd = 8 * j + 4 * hh + i;
        float* po = p.part_o + (pb + (size_t)hd * p.nsplit) * kSfaDv;
#pragma unroll
        for (int nb = 0; nb < 16; ++nb) po[32 * nb + c] = o[nb][4 * j + i];
      }
    if (hh == 0) {
      float* pm = p.part_ml + (pb + (size_t)c * p.nsplit) * 2;
      pm[0] = m2;
      pm[1] = lt;
    }
  }
}

// Reference computation of one (query, head), fp32 throughout, by the calling workgroup of
// NTR threads: z_j over the selected rows, the softmax, then O.  LDS: the caller's `ws`.
struct RefSmem {
  float qs[1024];
  float z[kMaxTopK];
  int64_t rws[kMaxTopK];
  float red[16];
};
template <int NTR>
__device__ void reference_head(const SfaParams& p, int t, int h, RefSmem& ws) {
  const int tid = threadIdx.x;
  const int seq = p.q_seq[t];
  const bool f32 = p.dtype == kDtF32;
  for (int d = tid; d < p.dqk; d += NTR) {
    const size_t qi = ((size_t)t * p.H + h) * p.dqk + d;
    ws.qs[d] = f32 ? ((const float*)p.q)[qi] : bf16_bits_to_f32(((const uint16_t*)p.q)[qi]);
  }
  __syncthreads();
  auto kvat = [&](int64_t row, int d) -> float {
    const size_t i = (size_t)row * p.dqk + d;
    return f32 ? ((const float*)p.kv)[i] : bf16_bits_to_f32(((const uint16_t*)p.kv)[i]);
  };
  float lmax = -INFINITY;
  for (int j = tid; j < p.K; j += NTR) {
    const int pos = p.idx[(size_t)t * p.K + j];
    float zz = -INFINITY;
    int64_t row = -1;
    if (pos >= 0) {
      row = pool_row(p.L, seq, pos);
      float acc = 0.f;
      for (int d = 0; d < p.dqk; ++d) acc = fmaf(ws.qs[d], kvat(row, d), acc);
      zz = acc * p.scale;
    }
    ws.z[j] = zz;
    ws.rws[j] = row;
    lmax = fmaxf(lmax, zz);
  }
  for (int off = 32; off >= 1; off >>= 1) lmax = fmaxf(lmax, __shfl_xor(lmax, off, 64));
  if ((tid & 63) == 0) ws.red[tid >> 6] = lmax;
  __syncthreads();
  float M = ws.red[0];
  for (int w = 1; w < NTR / 64; ++w) M = fmaxf(M, ws.red[w]);
  __syncthreads();
  float ls = 0.f;
  for (int j = tid; j < p.K; j += NTR) {
    const float e = (M == -INFINITY || ws.rws[j] < 0) ? 0.f : expf(ws.z[j] - M);
    ws.z[j] = e;
    ls += e;
  }
  for (int off = 32; off >= 1; off >>= 1) ls += __shfl_xor(ls, off, 64);
  if ((tid & 63) == 0) ws.red[8 + (tid >> 6)] = ls;
  __syncthreads();
  float L = 0.f;
  for (int w = 0; w < NTR / 64; ++w) L += ws.red[8 + w];
  const float inv = L > 0.f ? 1.f / L : 0.f;
  for (int d = tid; d < p.dv; d += NTR) {
    float acc = 0.f;
    for (int j = 0; j < p.K; ++j)
      if (ws.rws[j] >= 0) acc = fmaf(ws.z[j], kvat(ws.rws[j], d), acc);
    const size_t oi = ((size_t)t * p.H + h) * p.dv + d;
    if (f32) ((float*)p.out)[oi] = acc * inv;
    else ((uint16_t*)p.out)[oi] = (uint16_t)f32_to_bf16_bits(acc * inv);
  }
  if (p.lse && tid == 0) p.lse[(size_t)t * p.H + h] = L > 0.f ? M + logf(L) : -INFINITY;
}

// Reference mode: one workgroup per (query, head).
constexpr int kRefThreads = 256;
__global__ __launch_bounds__(kRefThreads) void sfa_reference_kernel(SfaParams p) {
  __shared__ RefSmem ws;
  reference_head<kRefThreads>(p, blockIdx.y, blockIdx.x, ws);
}

// Log-sum-exp weighted merge of the index-list slices, one workgroup per (head, query), one
// float4 of the 512 output dims per thread.  A head flagged by the MFMA kernel (scores far
// above its exponent reference) is recomputed by the reference method instead; the flag is
// cleared for the next call.
constexpr int kCombineThreads = 128;
__global__ __launch_bounds__(kCombineThreads) void sfa_combine_kernel(SfaParams p) {
  __shared__ RefSmem ws;
  const int h = blockIdx.x, t = blockIdx.y;
  uint32_t* flag = p.flags + (size_t)t * p.H + h;
  if (*flag) {
    reference_head<kCombineThreads>(p, t, h, ws);
    __syncthreads();
    if (threadIdx.x == 0) *flag = 0u;
    return;
  }
  if (p.nsplit == 1) return;
  const int ns = p.nsplit;
  const size_t base = ((size_t)t * p.H + h) * ns;
  const float* pm = p.part_ml + base * 2;
  float M = -INFINITY;
  for (int r = 0; r < ns; ++r) M = fmaxf(M, pm[2 * r]);
  float L = 0.f;
  for (int r = 0; r < ns; ++r) L += M == -INFINITY ? 0.f : exp2f(pm[2 * r] - M) * pm[2 * r + 1];
  const float inv = L > 0.f ? 1.f / L : 0.f;
  const int d = 4 * threadIdx.x;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const float* po = p.part_o + base * kSfaDv + d;
#pragma unroll 4
  for (int r = 0; r < ns; ++r) {
    const float w = M == -INFINITY ? 0.f : exp2f(pm[2 * r] - M) * inv;
    const f32x4 v = *(const f32x4*)(po + (size_t)r * kSfaDv);
    acc += w * v;
  }
  uint16_t* out = (uint16_t*)p.out + ((size_t)t * p.H + h) * kSfaDv + d;
  const uint32_t lo = f32_to_bf16_bits(acc[0]) | (f32_to_bf16_bits(acc[1]) << 16);
  const uint32_t hi = f32_to_bf16_bits(acc[2]) | (f32_to_bf16_bits(acc[3]) << 16);
  *(u32x2*)out = u32x2{lo, hi};
  if (p.lse && threadIdx.x == 0) p.lse[(size_t)t * p.H + h] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
}

}  // namespace

SfaPlan plan_sfa(int32_t T, int32_t H, int32_t K, int32_t dv, bool fast_path) {
  SfaPlan pl{};
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  if (!fast_path) {
    pl.heads_per_wg = 1;
    pl.n_hg = H;
    pl.rows_per_split = K;
    pl.nsplit = 1;
  } else {
    // One workgroup per CU holds the output accumulators of its heads in registers.  When
    // the (query, head group) pairs alone do not fill the chip, the index list is split into
    // slices (at most 1024 rows each) until about one workgroup per CU runs.
    const bool wide = (int64_t)T * (H / 128) >= 256;
    pl.heads_per_wg = (H % 128 == 0) ? 128 : (H % 96 == 0) ? 96 : (H % 64 == 0) ? 64 : 32;
    pl.n_hg = H / pl.heads_per_wg;
    const int64_t max_ns = (K + kTileRows - 1) / kTileRows;
    int64_t ns = 1;
    if (!wide) {
      const int64_t want = 256;
      ns = (want + (int64_t)T * pl.n_hg - 1) / ((int64_t)T * pl.n_hg);
      if (const char* e = getenv("DSA_SFA_SPLITS")) ns = atoll(e) > 0 ? atoll(e) : ns;
      const int64_t min_ns = (K + 1023) / 1024;
      if (ns < min_ns) ns = min_ns;
    }
    if (ns > max_ns) ns = max_ns;
    int64_t rps = (K + ns - 1) / ns;
    rps = (rps + kTileRows - 1) / kTileRows * kTileRows;
    pl.rows_per_split = (int32_t)rps;
    pl.nsplit = (int32_t)((K + rps - 1) / rps);
  }
  size_t off = 0;
  pl.off_counters = off;
  off = al(off + 16);
  pl.off_flags = off;
  off = al(off + (size_t)T * H * 4);
  pl.off_part = off;
  if (pl.nsplit > 1) off = al(off + (size_t)T * H * pl.nsplit * dv * 4);
  pl.off_ml = off;
  if (pl.nsplit > 1) off = al(off + (size_t)T * H * pl.nsplit * 8);
  pl.bytes = off;
  return pl;
}

hipError_t launch_sfa(const SfaParams& p, bool fast_path, hipStream_t stream) {
  if (!fast_path) {
    hipLaunchKernelGGL(sfa_reference_kernel, dim3(p.H, p.T), dim3(kRefThreads), 0, stream, p);
    return hipGetLastError();
  }
  // one workgroup per (query, slice) pair rounded up to whole groups of 8, times head groups
  const int pairs = (p.T * p.nsplit + 7) / 8 * 8;
  const dim3 grid(pairs * p.n_hg);
  switch (p.heads_per_wg) {
    case 128: hipLaunchKernelGGL(sfa_mfma_kernel<4>, grid, dim3(256), 0, stream, p); break;
    case 96: hipLaunchKernelGGL(sfa_mfma_kernel<3>, grid, dim3(192), 0, stream, p); break;
    case 64: hipLaunchKernelGGL(sfa_mfma_kernel<2>, grid, dim3(128), 0, stream, p); break;
    default: hipLaunchKernelGGL(sfa_mfma_kernel<1>, grid, dim3(64), 0, stream, p); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // merges the slices, and recomputes any flagged head (with one slice it only checks flags)
  hipLaunchKernelGGL(sfa_combine_kernel, dim3(p.H, p.T), dim3(kCombineThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace dsa
