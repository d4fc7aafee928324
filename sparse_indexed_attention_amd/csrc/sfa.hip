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
//   * Gather: tiles of 32 rows land in LDS through direct-to-LDS loads into three buffers (tiles
//     i+1 and i+2 stream in while tile i is computed).  LDS rows are 73 sixteen-byte chunks (one of
//     padding): with that odd stride both the MFMA reads of 16 rows at one column and the
//     transposing reads of 4 rows x 2 chunks touch distinct banks.  The pool rows of the slice
//     are resolved once, into LDS.
//   * Each wave holds 32 heads.  S^T = R . Q^T on v_mfma_f32_32x32x16_bf16: tile rows are the
//     A operand and the wave's queries (registers) the B operand, so a lane column is a head.
//   * Softmax in the exp2 domain without rescaling: a head's exponent reference is set by its
//     first live tile and never moved, so the output accumulators are never rescaled; a head
//     whose scores climb more than 64 above that reference is flagged and recomputed by the
//     reference method (fp32) after the attention kernel.
//   * O += P . V on the same MFMA, split by output dims: the head-owner waves write their
//     probabilities (bf16, in the accumulator's k order, so the k order of the contraction is
//     permuted to the rows each lane holds) to a small P tile in LDS; every wave then computes
//     O for all the workgroup's heads over its own 512/NW output dims, with P as the A operand
//     and V straight from the row-major tile through the transposing LDS read
//     ds_read_b64_tr_b16, which gathers one dim of four rows into a lane.
//   * Slices of the index list are merged by a log-sum-exp weighted combine kernel.
//   * Small decode batches take a 64-head variant (sfa_mfma64_kernel, below) that halves the
//     slices a query needs.
//   * fp8 latent rows (656 bytes: four 128-column tiles of e4m3 codes with power-of-two
//     scales, the rope columns in bf16): tiles of fp8 rows stream into four smaller LDS
//     staging buffers (three tiles in flight instead of two), and the contractions widen their
//     operands from the staged tile as they read them, with v_cvt_scalef32_pk_bf16_fp8,
//     exactly (a code times a power of two is a bf16 value); see the fp8 tile loop.
// Reference path (fp32 storage or other shapes): one workgroup per (query, head), fp32.

#include <cstdlib>

#include "dsa_internal.hpp"

namespace dsa {
namespace {

typedef int32_t v2i32 __attribute__((ext_vector_type(2)));

constexpr int kTileRows = 32;
constexpr int kRowBytes = kSfaDqk * 2;                   // 1152
constexpr int kRowChunks = kRowBytes / 16;               // 72 sixteen-byte chunks per row
constexpr int kLdsChunks = kRowChunks + 1;               // LDS row stride, in chunks
constexpr int kTileSlots = kTileRows * kLdsChunks;       // 2336
constexpr int kTileBytes = kTileSlots * 16;              // 37376
constexpr int kTileLoads = (kTileSlots + 63) / 64;       // 37 direct-to-LDS loads per tile
constexpr int kTileBufs = 3;                             // LDS tile buffers (two tiles ahead)
constexpr int kRowChunksF8 = kSfaRowF8 / 16;             // 41 sixteen-byte chunks per fp8 row
constexpr int kTileSlotsF8 = kTileRows * kRowChunksF8;   // 1312 (rows packed, no padding)
constexpr int kTileBytesF8 = kTileSlotsF8 * 16;          // 20992
constexpr int kTileLoadsF8 = (kTileSlotsF8 + 63) / 64;   // 21
constexpr int kStageBufs = 4;                            // fp8 staging buffers
constexpr int kBtLds = 4096;                             // block-table entries staged in LDS
constexpr int kPStride = 80;                             // bytes per head row of the shared P tile
constexpr int kPStride32 = 144;                          // ... in fp32 (fp8 rows: 128 bytes + 16)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Byte offset in a tile of chunk c of row r.
__device__ __forceinline__ int tile_off(int r, int c) { return 16 * (r * kLdsChunks + c); }

// 8 e4m3 codes (little-endian in r) times the power-of-two scale sc, as bf16: exact.
__device__ __forceinline__ bf16x8 widen_fp8x8(u32x2 r, float sc) {
  const bf16x2 a0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.x, sc, false);
  const bf16x2 a1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.x, sc, true);
  const bf16x2 a2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.y, sc, false);
  const bf16x2 a3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.y, sc, true);
  return bf16x8{a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
}

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
// 4 bytes per active lane from a per-lane global address into LDS at lds + 4 * lane.
__device__ __forceinline__ void load4_to_lds(const void* gaddr, uint32_t lds_in) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_in);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :: "v"(gaddr), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop

// Pool row of the slots of tile row rr in load I of a tile (the load fills slots 64 I ..
// 64 I + 63), from trow, whose lane l holds the pool row of the tile's row l % 32.  A load's
// slots span at most two rows (three for the packed fp8 rows), taken with readlane: reading the
// row from LDS per load instead costs an LDS round trip per load, each waited for before its
// load (the loads' asm keeps later memory accesses behind it) and queued behind the other
// waves' operand reads; on chunked prefill the attention kernel runs 3% faster this way.  (The
// 64-head decode kernel keeps the per-load read: the readlanes measured slower there.)
template <bool F8>
__device__ __forceinline__ int tile_pool_row(int32_t trow, int I, int rr) {
  constexpr int per_row = F8 ? kRowChunksF8 : kLdsChunks;
  const int r0 = (64 * I) / per_row;                 // first row of load I (wave-uniform)
  const int ra = __builtin_amdgcn_readlane(trow, r0);
  const int rb = __builtin_amdgcn_readlane(trow, min(r0 + 1, kTileRows - 1));
  if constexpr (F8) {
    const int rc = __builtin_amdgcn_readlane(trow, min(r0 + 2, kTileRows - 1));
    return rr == r0 ? ra : rr == r0 + 1 ? rb : rc;
  } else {
    return rr == r0 ? ra : rb;
  }
}

// Row of the 32x32 MFMA accumulator element r held by lane half h (lane column = l & 31).
__device__ __forceinline__ int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// Max / sum of a value and the one held by the lane 32 apart: v_permlane32_swap exchanges the
// halves, one of its two results is the lane's own value and the other its partner's.
__device__ __forceinline__ float xhalf_max(float v) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float xhalf_sum(float v) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

template <int NW, bool F8>
__global__ __launch_bounds__(NW * 64, 1) void sfa_mfma_kernel(SfaParams p) {
  constexpr int NTS = NW * 64;
  constexpr int TLOADS = F8 ? kTileLoadsF8 : kTileLoads;
  constexpr int LPW = (TLOADS + NW - 1) / NW;      // loads per wave per tile (at most)
  constexpr int LPW_MIN = TLOADS / NW;              // ... and at least
  // bf16 tiles (fp8 rows: one, filled from the staging buffers)
  __shared__ __attribute__((aligned(16))) uint8_t tiles[F8 ? 1 : kTileBufs][F8 ? 16 : kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t stage[F8 ? kStageBufs : 1][F8 ? kTileBytesF8 : 16];
  __shared__ int32_t rows[kMaxTopK];                // pool row of each slice entry, -1 if none
  __shared__ int32_t bt_lds[kBtLds];                // the sequence's block-table row
  __shared__ __attribute__((aligned(16))) float hv[NW * 32];   // per-head values
  __shared__ __attribute__((aligned(16))) uint8_t plds[NW * 32 * (F8 ? kPStride32 : kPStride)];   // P of the tile

  // workgroup -> (query, head group, slice); consecutive workgroups go to different XCDs, so
  // the head groups of one (query, slice) are placed 8 apart and share an XCD's L2
  const int wg = blockIdx.x;
  const int xcd = wg & 7, qq = wg >> 3;
  const int hg = qq % p.n_hg;
  const int cc = (qq / p.n_hg) * 8 + xcd;
  if (cc >= p.T * p.nsplit) return;
  const int t = cc / p.nsplit, r = cc - t * p.nsplit;
  tl_stamp(p.tl, kTlSfa, kTlStart);
  tl_clock(p.tl, kTlSfa, kTlClockStart);
  tl_put(p.tl, kTlSfa, kTlItem, ((uint64_t)t << 16) | ((uint32_t)hg << 8) | (uint32_t)r);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5, c = lane & 31;          // lane half, lane column
  const int hw = hg * NW + wave;                    // this wave's group of 32 heads
  const int h0 = hw * 32;
  const int seq = p.q_seq[t];
  const int j0 = r * p.rows_per_split;
  const int nrows = min(p.K, j0 + p.rows_per_split) - j0;
  const int ntiles = (nrows + kTileRows - 1) / kTileRows;

  // Pool rows of the slice.  The positions and the sequence's whole block-table row (when it
  // fits in LDS) are requested together, so the lookup costs one memory round trip; the first
  // tiles are issued right after it, and the queries after those, so that the query reads
  // overlap the row gather.
  constexpr int UI = kMaxTopK / NTS;                 // slice entries per thread (at most)
  int32_t posr[UI];
  {
    const int32_t* idx = p.idx + (size_t)t * p.K + j0;
#pragma unroll
    for (int u = 0; u < UI; ++u) {
      const int i = tid + u * NTS;
      posr[u] = i < nrows ? idx[i] : -1;
    }
  }
  const bool stage_bt = p.L.bt != nullptr && p.L.bt_stride <= kBtLds;
  if (stage_bt) {
    const int32_t* btrow = p.L.bt + (size_t)seq * p.L.bt_stride;
    for (int c0 = 64 * wave; c0 < p.L.bt_stride; c0 += NTS)
      if (c0 + lane < p.L.bt_stride) load4_to_lds(btrow + c0 + lane, lds_u32(bt_lds + c0));
  }
  wait_vmcnt<0>();
  __syncthreads();
#pragma unroll
  for (int u = 0; u < UI; ++u) {
    const int i = tid + u * NTS;
    if (i < ntiles * kTileRows) {
      const int pos = posr[u];
      int32_t row = -1;
      if (pos >= 0) {
        if (stage_bt) {
          const int sh = p.L.bs_log2;
          row = (bt_lds[pos >> sh] << sh) | (pos & ((1 << sh) - 1));
        } else {
          row = (int32_t)pool_row(p.L, seq, pos);
        }
      }
      rows[i] = row;
    }
  }
  __syncthreads();

  // queries of this wave's 32 heads (lane holds head c, dims 16s + 8hh .. +7).  Issued after
  // the first tiles: the first read of them waits for every load issued before, which by
  // then are only the first tiles the attention step needs anyway.
  bf16x8 qk[36];
  auto load_queries = [&]() {
    const uint16_t* qb = (const uint16_t*)p.q + ((size_t)t * p.H + h0 + c) * kSfaDqk + 8 * hh;
#pragma unroll
    for (int s = 0; s < 36; ++s) qk[s] = *(const bf16x8*)(qb + 16 * s);
  };
  const uint8_t* kv = (const uint8_t*)p.kv;
  const uint8_t* zero = (const uint8_t*)p.zero;
  // This wave's share of tile `tile`: loads I = wave, wave + NW, ...; lane l of load I fills
  // chunk slot 64 I + l.  Rows without a position are filled from a zeroed global chunk, so
  // every load instruction has active lanes (a padding slot is at most one lane of 64) and
  // each wave issues the same number of loads for every tile: the vmcnt waits below count
  // on that.
  auto issue = [&](int tile, int buf) {
    uint8_t* tb = F8 ? stage[buf] : tiles[buf];
    // an opaque zero: the slot arithmetic below is redone per call instead of being hoisted
    // out of the tile loop into registers that the attention step needs
    int z0 = 0;
    asm volatile("" : "+v"(z0));
    const int32_t trow = rows[tile * kTileRows + (lane & 31)];   // the tile's pool rows
#pragma unroll
    for (int u = 0; u < LPW; ++u) {
      const int I = wave + NW * u;
      if (LPW != LPW_MIN && I >= TLOADS) break;
      const int P = 64 * I + lane + z0;
      if constexpr (F8) {
        // fp8 rows are packed in the staging buffer: slot P is chunk P % 41 of row P / 41
        const int rr = P / kRowChunksF8, ch = P - rr * kRowChunksF8;
        if (P < kTileSlotsF8) {
          const int row = tile_pool_row<F8>(trow, I, rr);
          load16_to_lds(row >= 0 ? kv + (size_t)row * kSfaRowF8 + 16 * ch : zero, lds_u32(tb + 1024 * I));
        }
      } else {
        const int rr = P / kLdsChunks, ch = P - rr * kLdsChunks;
        if (P < kTileSlots && ch < kRowChunks) {
          const int row = tile_pool_row<F8>(trow, I, rr);
          load16_to_lds(row >= 0 ? kv + (size_t)row * kRowBytes + 16 * ch : zero, lds_u32(tb + 1024 * I));
        }
      }
    }
  };
  const float scale2 = p.scale * kLog2e;

  // S^T = R . Q^T for the tile in `tb`, scaled to the exp2 domain, -inf for empty rows: lane
  // (hh, c) gets rows acc_row(e, hh) of head c.  The operand reads of the next four k steps
  // are issued before the MFMAs of the current four (scheduling fences keep that order); the
  // register file holds the queries and the output accumulators, so there is room for little
  // more.
  auto scores = [&](const uint8_t* tb, uint32_t valid, float (&z)[16]) {
    f32x16 sa = {};
    const uint8_t* ra = tb + tile_off(c, hh);
    bf16x8 a[2][4];
#pragma unroll
    for (int u = 0; u < 4; ++u) a[0][u] = *(const bf16x8*)(ra + 32 * u);
#pragma unroll
    for (int g = 0; g < 9; ++g) {
      if (g + 1 < 9) {
#pragma unroll
        for (int u = 0; u < 4; ++u) a[(g + 1) & 1][u] = *(const bf16x8*)(ra + 32 * (4 * (g + 1) + u));
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < 4; ++u) sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[g & 1][u], qk[4 * g + u], sa, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (valid == 0xffffffffu) {
#pragma unroll
      for (int e = 0; e < 16; ++e) z[e] = sa[e] * scale2;
    } else {
      const uint32_t mh = valid >> (4 * hh);
#pragma unroll
      for (int e = 0; e < 16; ++e)
        z[e] = (mh >> (8 * (e >> 2) + (e & 3))) & 1u ? sa[e] * scale2 : -INFINITY;
    }
  };

  // Exponent reference m2 per head: set by the head's first live tile and never moved, so the
  // output accumulators are never rescaled.  Probabilities exp2(z - m2) may exceed 1; up to
  // 2^64 bf16 operands and fp32 sums of 2^11 terms keep their full relative precision.  A
  // head whose scores pass m2 + 64 is flagged, and the combine kernel recomputes it with the
  // reference method.
  //
  // O += P . V is split by output dims: wave w owns dims [DW*w, DW*w + DW) of every head of
  // the workgroup, so each wave reads only its quarter of V from LDS (the transposing reads
  // move half the bytes per instruction of plain ones, and V was the largest LDS stream).
  // The probabilities computed by the head-owner waves are exchanged through a small LDS tile.
  constexpr int DW = kSfaDv / NW;                  // output dims per wave
  constexpr int NB = DW / 32;                      // 32-dim blocks per wave
  float m2 = -INFINITY, l = 0.f;
  f32x16 o[NW * NB];                               // [head block][dim block]
  bool over = false;
  // V operand for dims 32nb .. +31, k step kk: in each 16-lane group, lane i supplies row
  // 16kk + 8jj + 4hh + i/4, dims 32nb + 16(c/16) + 4(i%4) .. +3; the transposing read returns
  // dim 32nb + c of four consecutive rows
  const int vi = c & 15;
  const int vrow = 4 * hh + (vi >> 2);
  const int vdim = 16 * (c >> 4) + 4 * (vi & 3);
  auto attend = [&](int tile, const uint8_t* tb) {
    const uint32_t valid = (uint32_t)__ballot(rows[tile * kTileRows + c] >= 0);
    float z[16];
    scores(tb, valid, z);
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = fmaxf(mx, z[e]);
    mx = xhalf_max(mx);
    if (m2 == -INFINITY) m2 = mx;                // first live tile of this head (O, l are 0)
    over |= mx > m2 + 64.f;
    const bool live = m2 != -INFINITY;
    float pe[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      pe[e] = live ? __builtin_amdgcn_exp2f(z[e] - m2) : 0.f;
      l += pe[e];
    }
    // P as the A operand of k step kk: k slot 8hh + u is row 16kk + 8(u/4) + 4hh + u%4, i.e.
    // accumulator elements 8kk .. 8kk+7 as they stand.  Head row c of this wave goes to the
    // shared tile in that k order, 16 bytes per k step.
    {
      bf16x8 pw[2];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        pw[0][u] = (__bf16)pe[u];
        pw[1][u] = (__bf16)pe[8 + u];
      }
      uint8_t* prow = plds + (32 * wave + c) * kPStride + 16 * hh;
      *(bf16x8*)prow = pw[0];
      *(bf16x8*)(prow + 32) = pw[1];
    }
    __syncthreads();                             // every head's P is in the tile
    bf16x8 pa[NW][2];
#pragma unroll
    for (int hb = 0; hb < NW; ++hb)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        pa[hb][kk] = *(const bf16x8*)(plds + (32 * hb + c) * kPStride + 32 * kk + 16 * hh);
    auto vread = [&](int nb, s16x4 (&v)[4]) {
      const int dim = DW * wave + 32 * nb + vdim;
      const int cho = tile_off(0, dim >> 3) + 2 * (dim & 7);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        v[q] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(tb + tile_off(8 * q + vrow, 0) + cho));
    };
    s16x4 vb[2][4];
    vread(0, vb[0]);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      if (nb + 1 < NB) vread(nb + 1, vb[(nb + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      const s16x4* v = vb[nb & 1];
      bf16x8 b[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        b[kk] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v[2 * kk], v[2 * kk + 1], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int hb = 0; hb < NW; ++hb)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
          o[hb * NB + nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[hb][kk], b[kk], o[hb * NB + nb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

#pragma unroll
  for (int n = 0; n < NW * NB; ++n) o[n] = f32x16{};
  TlCycles tc;
  if constexpr (F8) {
    // fp8 rows: the contractions read the landed staging tile directly.  S^T: the A fragment
    // of row c and k step s < 32 is 8 codes (one 8-byte read) widened to bf16 with the row's
    // scale of tile s / 8 by v_cvt_scalef32_pk_bf16_fp8 (exact: a code times a power of two is a
    // bf16 value); steps 32..35 read the bf16 rope columns.  P . V: the value codes are widened
    // with scale 1 and each row's scale of the wave's dim tile multiplies P instead (a power of
    // two, exact in fp32), so P is exchanged in fp32 and rounded to bf16 once, per wave, after
    // its scaling.  The B fragments come from the 8-bit transposing read ds_read_b64_tr_b8: in
    // each 16-lane group g, lane 8h + i receives byte i of the 8-byte chunks that lanes
    // 16g + h + 2b (b = 0..7) address, so lane s of the group addresses k slot
    // 8(g / 2) + (s % 16) / 2 of the step at dims 16(g % 2) + 8(s % 2) of the block.
    static_assert(kStageBufs == 4 && 3 * LPW_MIN < 64, "waits below");
    auto attend8 = [&](int tile, const uint8_t* sb) {
      const uint32_t valid = (uint32_t)__ballot(rows[tile * kTileRows + c] >= 0);
      float z[16];
      {
        const uint8_t* ra = sb + c * kSfaRowF8;
        const f32x4 sc = *(const f32x4*)(ra + 640);
        f32x16 sa = {};
        u32x2 raw[2][4];
#pragma unroll
        for (int u = 0; u < 4; ++u) raw[0][u] = *(const u32x2*)(ra + 16 * u + 8 * hh);
#pragma unroll
        for (int g = 0; g < 8; ++g) {
          if (g + 1 < 8) {
#pragma unroll
            for (int u = 0; u < 4; ++u) raw[(g + 1) & 1][u] = *(const u32x2*)(ra + 16 * (4 * (g + 1) + u) + 8 * hh);
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int u = 0; u < 4; ++u)
            sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(widen_fp8x8(raw[g & 1][u], sc[g >> 1]), qk[4 * g + u], sa, 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        bf16x8 ar[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) ar[u] = *(const bf16x8*)(ra + 512 + 32 * u + 16 * hh);
#pragma unroll
        for (int u = 0; u < 4; ++u) sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ar[u], qk[32 + u], sa, 0, 0, 0);
        if (valid == 0xffffffffu) {
#pragma unroll
          for (int e = 0; e < 16; ++e) z[e] = sa[e] * scale2;
        } else {
          const uint32_t mh = valid >> (4 * hh);
#pragma unroll
          for (int e = 0; e < 16; ++e)
            z[e] = (mh >> (8 * (e >> 2) + (e & 3))) & 1u ? sa[e] * scale2 : -INFINITY;
        }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, z[e]);
      mx = xhalf_max(mx);
      if (m2 == -INFINITY) m2 = mx;
      over |= mx > m2 + 64.f;
      const bool live = m2 != -INFINITY;
      float pe[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        pe[e] = live ? __builtin_amdgcn_exp2f(z[e] - m2) : 0.f;
        l += pe[e];
      }
      {
        // head row c of this wave, k step kk, k slots 8 hh .. 8 hh + 7: floats 16 kk + 8 hh
        float* prow = (float*)(plds + (32 * wave + c) * kPStride32) + 8 * hh;
        *(f32x4*)prow = f32x4{pe[0], pe[1], pe[2], pe[3]};
        *(f32x4*)(prow + 4) = f32x4{pe[4], pe[5], pe[6], pe[7]};
        *(f32x4*)(prow + 16) = f32x4{pe[8], pe[9], pe[10], pe[11]};
        *(f32x4*)(prow + 20) = f32x4{pe[12], pe[13], pe[14], pe[15]};
      }
      __syncthreads();                           // every head's P is in the tile
      // this lane's source row for the transposing reads (k slot of step kk: + 16 kk)
      const int tg = lane >> 4, tu = (lane & 15) >> 1;
      const int trow = 8 * (tu >> 2) + 4 * (tg >> 1) + (tu & 3);
      const int tdim = 16 * (tg & 1) + 8 * (lane & 1);
      bf16x8 pa[NW][2];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int dim0 = DW * wave + 32 * nb;
        if ((nb & 3) == 0) {
          // P times the rows' scales of dim tile dim0 / 128 (k slot 8 hh + u of step kk is row
          // 16 kk + 8 (u / 4) + 4 hh + u % 4)
          const int tsc = 640 + 4 * (dim0 >> 7);
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            float vs[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
              vs[u] = *(const float*)(sb + (16 * kk + 8 * (u >> 2) + 4 * hh + (u & 3)) * kSfaRowF8 + tsc);
#pragma unroll
            for (int hb = 0; hb < NW; ++hb) {
              const float* pr = (const float*)(plds + (32 * hb + c) * kPStride32) + 16 * kk + 8 * hh;
              const f32x4 p0 = *(const f32x4*)pr, p1 = *(const f32x4*)(pr + 4);
#pragma unroll
              for (int u = 0; u < 4; ++u) {
                pa[hb][kk][u] = (__bf16)(p0[u] * vs[u]);
                pa[hb][kk][4 + u] = (__bf16)(p1[u] * vs[4 + u]);
              }
            }
          }
        }
        bf16x8 b[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const v2i32 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (__attribute__((address_space(3))) v2i32*)(sb + (16 * kk + trow) * kSfaRowF8 + dim0 + tdim));
          b[kk] = widen_fp8x8(u32x2{(uint32_t)v.x, (uint32_t)v.y}, 1.f);
        }
#pragma unroll
        for (int hb = 0; hb < NW; ++hb)
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
            o[hb * NB + nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[hb][kk], b[kk], o[hb * NB + nb], 0, 0, 0);
      }
    };
    for (int i = 0; i < kStageBufs && i < ntiles; ++i) issue(i, i);
    load_queries();
    int buf = 0;
    for (int tile = 0; tile < ntiles; ++tile) {
      tc.mark();
      const int ahead = min(ntiles - 1 - tile, kStageBufs - 1);   // later tiles in flight
      if (ahead >= 3) wait_vmcnt<3 * LPW_MIN>();
      else if (ahead == 2) wait_vmcnt<2 * LPW_MIN>();
      else if (ahead == 1) wait_vmcnt<LPW_MIN>();
      else wait_vmcnt<0>();
      __syncthreads();                           // every wave's loads of `tile` have landed
      tc.waited();
      attend8(tile, stage[buf]);
      __syncthreads();                           // the staging buffer and the P tile are free
      tc.computed();
      if (tile + kStageBufs < ntiles) issue(tile + kStageBufs, buf);
      tc.issued();
      buf = buf == kStageBufs - 1 ? 0 : buf + 1;
    }
  } else {
  // Tiles stream through kTileBufs LDS buffers, kTileBufs - 1 of them ahead of the one being
  // computed.  (Issuing tile i + 2 after the barrier that opens tile i, which would save the
  // second barrier per tile, measured slower on chunked prefill: the gather needs the lead.)
  static_assert(kTileBufs == 3, "prologue below issues three tiles");
  if (ntiles > 0) issue(0, 0);
  if (ntiles > 1) issue(1, 1);
  if (ntiles > 2) issue(2, 2);
  load_queries();
  int buf = 0;
  for (int tile = 0; tile < ntiles; ++tile) {
    tc.mark();
    const int ahead = min(ntiles - 1 - tile, kTileBufs - 1);   // later tiles in flight
    if (ahead >= 2) wait_vmcnt<(2 * LPW_MIN < 63 ? 2 * LPW_MIN : 63)>();   // capped: waits longer
    else if (ahead == 1) wait_vmcnt<LPW_MIN>();
    else wait_vmcnt<0>();                        // this wave's loads of `tile` have landed
    __syncthreads();                             // ... and every other wave's
    tc.waited();
    attend(tile, tiles[buf]);
    __syncthreads();                             // the buffer and the P tile are free again
    tc.computed();
    if (tile + kTileBufs < ntiles) issue(tile + kTileBufs, buf);
    tc.issued();
    buf = buf == kTileBufs - 1 ? 0 : buf + 1;
  }
  }
  tl_stamp(p.tl, kTlSfa, kTlLoopDone);
  tl_clock(p.tl, kTlSfa, kTlClockEnd);
  tc.put(p.tl, kTlSfa, ntiles);

  // per-head totals: the two lane halves of a column hold disjoint rows of its head
  const float lt = xhalf_sum(l);
  if (hh == 0) hv[32 * wave + c] = lt > 0.f ? 1.f / lt : 0.f;
  const uint32_t flagword = (uint32_t)__ballot(over);   // bit c: head h0 + c
  __syncthreads();                                      // every head's 1 / l
  const int hgb = hg * 32 * NW;                         // first head of the workgroup
  // accumulator (hb, nb) element 4j + i of lane (hh, c): head hgb + 32hb + 8j + 4hh + i,
  // dim DW*wave + 32nb + c
  if (p.nsplit == 1) {
    uint16_t* out = (uint16_t*)p.out + ((size_t)t * p.H + hgb) * kSfaDv + DW * wave + c;
#pragma unroll
    for (int hb = 0; hb < NW; ++hb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 inv = *(const f32x4*)&hv[32 * hb + 8 * j + 4 * hh];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int hd = 32 * hb + 8 * j + 4 * hh + i;
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            out[hd * kSfaDv + 32 * nb] = __builtin_bit_cast(uint16_t, (__bf16)(o[hb * NB + nb][4 * j + i] * inv[i]));
        }
      }
    if (p.lse && hh == 0)
      p.lse[(size_t)t * p.H + h0 + c] = lt > 0.f ? (m2 + log2f(lt)) * kLn2 : -INFINITY;
  } else {
    // Partial of this slice: O / l in fp16, stored as the accumulators lie in the registers,
    // 32 records of 1 KB (16 bytes per lane) per (query, head group, slice, wave).  Record
    // (hb*4 + j)*(NB/2) + np of lane (hh, c) holds heads 32hb + 8j + 4hh + i (i < 4) at dims
    // DW*wave + 32(2np + s) + c (s < 2), value 4s + i.  Record rec of (query, head group,
    // wave) for slice r lies at ((qhw * NREC + rec) * nsplit + r) KB: the slices of one record
    // are adjacent, so the merge reads them 1 KB apart (with the slice outermost, 32 to 128 KB
    // apart, the merge read measured slower)
    constexpr int NREC = NW * 4 * (NB / 2);
    uint8_t* po = (uint8_t*)p.part_o +
                  ((((size_t)t * p.n_hg + hg) * NW + wave) * NREC * p.nsplit + r) * 1024 + 16 * lane;
#pragma unroll
    for (int hb = 0; hb < NW; ++hb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 inv = *(const f32x4*)&hv[32 * hb + 8 * j + 4 * hh];
#pragma unroll
        for (int np = 0; np < NB / 2; ++np) {
          uint32_t w[4];
#pragma unroll
          for (int sd = 0; sd < 2; ++sd)
#pragma unroll
            for (int i = 0; i < 4; i += 2) {
              const _Float16 a = (_Float16)(o[hb * NB + 2 * np + sd][4 * j + i] * inv[i]);
              const _Float16 b = (_Float16)(o[hb * NB + 2 * np + sd][4 * j + i + 1] * inv[i + 1]);
              w[2 * sd + i / 2] = (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
            }
          *(u32x4*)(po + (size_t)((hb * 4 + j) * (NB / 2) + np) * p.nsplit * 1024) = u32x4{w[0], w[1], w[2], w[3]};
        }
      }
    if (hh == 0) {
      float* pm = p.part_ml + (((size_t)t * p.H + h0 + c) * p.nsplit + r) * 2;
      pm[0] = m2;
      pm[1] = lt;
    }
  }
  tl_stamp(p.tl, kTlSfa, kTlWritten);
  if (lane == 0) p.flags[((size_t)t * (p.H / 32) + hw) * p.nsplit + r] = flagword;
}

// Decode variant: a workgroup owns (query, group of 64 heads, slice of the index list) with
// four waves, so a decode batch needs half the slices (and half the partial outputs) of the
// 128-head workgroup for the same number of workgroups, and each reads half the queries.
//   * Tiles are taken in pairs.  QK^T: wave w scores tile (w >> 1) of the pair for heads
//     32 (w & 1) .. +31 of the group, exactly as above (tile rows the A operand, the wave's
//     queries the B operand).  The two waves of a head half exchange their tile maxima through
//     LDS, so both use the same exponent reference for the head (set by the first pair with a
//     live row, never moved; heads that climb more than 64 above it are flagged).
//   * P.V: wave w owns output dims 128 w .. +127 of all 64 heads over the pair's 64 rows
//     (probabilities from the shared P tile, values through the transposing LDS read).
//   * Four tile buffers: two pairs in flight.  The sequence's block-table row is staged in the
//     last buffer before any tile is loaded, and the workgroup's query rows in the last two
//     (while pair 0 lands) before pair 1 is.
//   * Slices write O / l in fp16 in the record format of the 128-head kernel with two head
//     blocks per wave (16 KB per wave), and (m, l) per head; the combine kernel merges them.
constexpr int kRows64 = 512;                           // most slice entries of the decode variant
constexpr int kPStride64 = 144;                        // bytes per head row of its P tile (64 rows)
constexpr int kPStride64F = 272;                       // ... in fp32 (fp8 rows: 256 bytes + 16)
// F8: fp8 latent rows, read and widened as in the 128-head kernel's fp8 tile loop (the rows'
// value scales folded into an fp32 P tile, the V fragments from the 8-bit transposing read).
// Its smaller buffers lie in one region [buffer 0 | buffer 1 | P tile | spare | buffer 2 |
// buffer 3] whose first 74,752 bytes take the padded query rows, so there pair 0 goes into
// buffers 2 and 3 and pair 1 into 0 and 1.
template <bool F8>
__global__ __launch_bounds__(256, 1) void sfa_mfma64_kernel(SfaParams p) {
  constexpr int NW = 4, NTS = 256;
  constexpr int TL = F8 ? kTileLoadsF8 : kTileLoads;
  constexpr int LPW = (TL + NW - 1) / NW, LPW_MIN = TL / NW;
  constexpr int kBufs = 4;
  constexpr int TB = F8 ? kTileBytesF8 : kTileBytes;
  constexpr int PS = F8 ? kPStride64F : kPStride64;
  constexpr int QTILE = 2 * kTileBytes;                      // 64 padded bf16 query rows
  constexpr int LO = 2 * TB + 64 * PS;                       // F8: buffers 0, 1 and the P tile
  constexpr int HI = F8 ? (LO > QTILE ? LO : QTILE) : LO;    // F8: start of buffer 2
  constexpr int REGION = F8 ? HI + 2 * TB : kBufs * TB + 64 * PS;
  __shared__ __attribute__((aligned(16))) uint8_t region[REGION];
  __shared__ int32_t rows[kRows64];
  __shared__ float xmax[NW][32], xsum[NW][32];
  __shared__ uint32_t xover[NW];
  __shared__ __attribute__((aligned(16))) float hv[64];
  static_assert(REGION + 4 * kRows64 + 2 * NW * 32 * 4 + 16 + 256 <= 163840, "LDS");
  static_assert(TB >= 4 * kBtLds, "block-table row staged in a tile buffer");
  // tile buffer b, the P tile, the query rows' landing place, and the buffers of pair pr
  auto tbuf = [&](int b) -> uint8_t* {
    if constexpr (F8) return region + (b < 2 ? b * TB : HI + (b - 2) * TB);
    else return region + b * TB;
  };
  uint8_t* const plds = F8 ? region + 2 * TB : region + kBufs * TB;
  uint8_t* const qland = F8 ? region : region + 2 * TB;
  auto pair_buf = [](int pr) { return F8 ? 2 * ((pr + 1) & 1) : 2 * (pr & 1); };

  // workgroup -> (query, head group, slice): the head groups of one (query, slice) are 8
  // apart, so consecutive workgroup numbers place them on one XCD, sharing its L2 for the rows
  const int wg = blockIdx.x;
  const int xcd = wg & 7, qq = wg >> 3;
  const int hg = qq % p.n_hg;
  const int cc = (qq / p.n_hg) * 8 + xcd;
  if (cc >= p.T * p.nsplit) return;
  const int t = cc / p.nsplit, r = cc - t * p.nsplit;
  tl_stamp(p.tl, kTlSfa, kTlStart);
  tl_clock(p.tl, kTlSfa, kTlClockStart);
  tl_put(p.tl, kTlSfa, kTlItem, ((uint64_t)t << 16) | ((uint32_t)hg << 8) | (uint32_t)r);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5, c = lane & 31;
  const int hq = wave & 1, par = wave >> 1;        // QK^T: head half, tile of the pair
  const int h0 = hg * 64 + hq * 32;                // first of this wave's QK^T heads
  const int seq = p.q_seq[t];
  const int j0 = r * p.rows_per_split;
  const int nrows = min(p.K, j0 + p.rows_per_split) - j0;
  const int ntiles = (nrows + kTileRows - 1) / kTileRows;
  const int npairs = (ntiles + 1) >> 1;

  // pool rows of the slice (one memory round trip: positions and the block-table row together)
  int32_t posr[kRows64 / NTS];
  {
    const int32_t* idx = p.idx + (size_t)t * p.K + j0;
#pragma unroll
    for (int u = 0; u < kRows64 / NTS; ++u) {
      const int i = tid + u * NTS;
      posr[u] = i < nrows ? idx[i] : -1;
    }
  }
  int32_t* bt_lds = (int32_t*)tbuf(kBufs - 1);
  const bool stage_bt = p.L.bt != nullptr && p.L.bt_stride <= kBtLds;
  if (stage_bt) {
    const int32_t* btrow = p.L.bt + (size_t)seq * p.L.bt_stride;
    for (int c0 = 64 * wave; c0 < p.L.bt_stride; c0 += NTS)
      if (c0 + lane < p.L.bt_stride) load4_to_lds(btrow + c0 + lane, lds_u32(bt_lds + c0));
  }
  wait_vmcnt<0>();
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kRows64 / NTS; ++u) {
    const int i = tid + u * NTS;
    if (i < 2 * npairs * kTileRows) {
      const int pos = posr[u];
      int32_t row = -1;
      if (pos >= 0) {
        if (stage_bt) {
          const int sh = p.L.bs_log2;
          row = (bt_lds[pos >> sh] << sh) | (pos & ((1 << sh) - 1));
        } else {
          row = (int32_t)pool_row(p.L, seq, pos);
        }
      }
      rows[i] = row;
    }
  }
  __syncthreads();                                 // rows ready; the staged block table is free
  tl_stamp(p.tl, kTlSfa, kTlRows);

  const uint8_t* kv = (const uint8_t*)p.kv;
  const uint8_t* zero = (const uint8_t*)p.zero;
  // this wave's share of tile `tile` (see the 128-head kernel): rows without a position load
  // from a zeroed chunk, so every wave issues the same number of loads per tile
  auto issue = [&](int tile, int buf) {
    uint8_t* tb = tbuf(buf);
    int z0 = 0;
    asm volatile("" : "+v"(z0));
#pragma unroll
    for (int u = 0; u < LPW; ++u) {
      const int I = wave + NW * u;
      if (LPW != LPW_MIN && I >= TL) break;
      const int P = 64 * I + lane + z0;
      if constexpr (F8) {
        const int rr = P / kRowChunksF8, ch = P - rr * kRowChunksF8;   // packed rows
        if (P < kTileSlotsF8) {
          const int row = rows[tile * kTileRows + rr];
          load16_to_lds(row >= 0 ? kv + (size_t)row * kSfaRowF8 + 16 * ch : zero, lds_u32(tb + 1024 * I));
        }
      } else {
        const int rr = P / kLdsChunks, ch = P - rr * kLdsChunks;
        if (P < kTileSlots && ch < kRowChunks) {
          const int row = rows[tile * kTileRows + rr];
          load16_to_lds(row >= 0 ? kv + (size_t)row * kRowBytes + 16 * ch : zero, lds_u32(tb + 1024 * I));
        }
      }
    }
  };
  auto issue_pair = [&](int pr) {
    issue(2 * pr, pair_buf(pr));
    issue(2 * pr + 1, pair_buf(pr) + 1);
  };
  issue_pair(0);
  bf16x8 qk[36];
  // The workgroup's 64 query rows (73.7 KB, contiguous) land as one 64-row tile in the padded
  // row layout (in buffers 2 and 3; with fp8 rows in the front of the region), behind pair 0's
  // tiles; each wave then reads its 32 heads' fragments from there.  Two waves share each head
  // half, so loading the fragments from global memory directly would fetch every query twice.
  // Pair 1 goes into the landing place once every wave has its fragments.  (Requesting the
  // query rows first, so that pair 1 could follow sooner, measured the same: a workgroup's
  // time is set by the bytes it brings in, not their order.)
  {
    const uint8_t* qrows = (const uint8_t*)p.q + ((size_t)t * p.H + hg * 64) * kRowBytes;
    constexpr int QLOADS = 2 * kTileSlots / 64;    // 73: 64 rows of 73 slots
    static_assert(2 * kTileSlots % 64 == 0, "query tile");
    for (int I = wave; I < QLOADS; I += NW) {
      const int P = 64 * I + lane;
      const int rr = P / kLdsChunks, ch = P - rr * kLdsChunks;
      if (ch < kRowChunks) load16_to_lds(qrows + (size_t)rr * kRowBytes + 16 * ch, lds_u32(qland + 1024 * I));
    }
  }
  wait_vmcnt<0>();
  __syncthreads();                                 // pair 0 and the query tile have landed
  tl_stamp(p.tl, kTlSfa, kTlFirstTile);
  {
    const uint8_t* qr = qland + tile_off(32 * hq + c, hh);   // head 32 hq + c, dims 8 hh + 16 s
#pragma unroll
    for (int s = 0; s < 36; ++s) qk[s] = *(const bf16x8*)(qr + 32 * s);
  }
  __syncthreads();                                 // every wave holds its fragments
  tl_stamp(p.tl, kTlSfa, kTlQueries);
  if (npairs > 1) issue_pair(1);

  const float scale2 = p.scale * kLog2e;
  float m2 = -INFINITY, l = 0.f;
  bool over = false;
  f32x16 o[2][4];                                  // [head block][32-dim block of this wave]
#pragma unroll
  for (int hb = 0; hb < 2; ++hb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) o[hb][nb] = f32x16{};
  const int vi = c & 15;
  const int vrow = 4 * hh + (vi >> 2);
  const int vdim = 16 * (c >> 4) + 4 * (vi & 3);

  TlCycles tc;
  for (int pr = 0; pr < npairs; ++pr) {
    const int b0 = pair_buf(pr);
    // Pairs 0 and 1 are issued before the loop, pair pr + 1 (pr >= 1) right after pair pr
    // opens: so only at pair 0 is a later pair in flight while waiting.
    tc.mark();
    if (pr == 0 && npairs > 1) wait_vmcnt<(2 * LPW_MIN < 63 ? 2 * LPW_MIN : 63)>();
    else wait_vmcnt<0>();
    __syncthreads();                               // every wave's loads of pair pr have landed,
                                                   // and every wave is done with pair pr - 1
    tc.waited();
    if (pr >= 1 && pr + 1 < npairs) issue_pair(pr + 1);   // into pair pr - 1's buffers
    // S^T for tile 2 pr + par, heads h0 .. h0 + 31
    const int tile = 2 * pr + par;
    const uint8_t* tb = tbuf(b0 + par);
    const uint32_t valid = (uint32_t)__ballot(rows[tile * kTileRows + c] >= 0);
    float z[16];
    {
      f32x16 sa = {};
      if constexpr (F8) {
        const uint8_t* ra = tb + c * kSfaRowF8;
        const f32x4 sc = *(const f32x4*)(ra + 640);
        u32x2 raw[2][4];
#pragma unroll
        for (int u = 0; u < 4; ++u) raw[0][u] = *(const u32x2*)(ra + 16 * u + 8 * hh);
#pragma unroll
        for (int g = 0; g < 8; ++g) {
          if (g + 1 < 8) {
#pragma unroll
            for (int u = 0; u < 4; ++u) raw[(g + 1) & 1][u] = *(const u32x2*)(ra + 16 * (4 * (g + 1) + u) + 8 * hh);
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int u = 0; u < 4; ++u)
            sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(widen_fp8x8(raw[g & 1][u], sc[g >> 1]), qk[4 * g + u], sa, 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        bf16x8 ar[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) ar[u] = *(const bf16x8*)(ra + 512 + 32 * u + 16 * hh);
#pragma unroll
        for (int u = 0; u < 4; ++u) sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ar[u], qk[32 + u], sa, 0, 0, 0);
      } else {
      const uint8_t* ra = tb + tile_off(c, hh);
      bf16x8 a[2][4];
#pragma unroll
      for (int u = 0; u < 4; ++u) a[0][u] = *(const bf16x8*)(ra + 32 * u);
#pragma unroll
      for (int g = 0; g < 9; ++g) {
        if (g + 1 < 9) {
#pragma unroll
          for (int u = 0; u < 4; ++u) a[(g + 1) & 1][u] = *(const bf16x8*)(ra + 32 * (4 * (g + 1) + u));
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < 4; ++u) sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[g & 1][u], qk[4 * g + u], sa, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      }
      const uint32_t mh = valid >> (4 * hh);
#pragma unroll
      for (int e = 0; e < 16; ++e)
        z[e] = (mh >> (8 * (e >> 2) + (e & 3))) & 1u ? sa[e] * scale2 : -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = fmaxf(mx, z[e]);
    mx = xhalf_max(mx);
    if (hh == 0) xmax[wave][c] = mx;
    __syncthreads();                               // both tiles' maxima of every head
    mx = fmaxf(mx, xmax[wave ^ 2][c]);
    if (m2 == -INFINITY) m2 = mx;                  // first pair with a live row of this head
    over |= mx > m2 + 64.f;
    const bool live = m2 != -INFINITY;
    if constexpr (F8) {
      float pe[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        pe[e] = live ? __builtin_amdgcn_exp2f(z[e] - m2) : 0.f;
        l += pe[e];
      }
      // head row 32 hq + c, k steps 2 par and 2 par + 1: floats 16 k + 8 hh .. + 7
      float* prow = (float*)(plds + (32 * hq + c) * PS) + 32 * par + 8 * hh;
      *(f32x4*)prow = f32x4{pe[0], pe[1], pe[2], pe[3]};
      *(f32x4*)(prow + 4) = f32x4{pe[4], pe[5], pe[6], pe[7]};
      *(f32x4*)(prow + 16) = f32x4{pe[8], pe[9], pe[10], pe[11]};
      *(f32x4*)(prow + 20) = f32x4{pe[12], pe[13], pe[14], pe[15]};
    } else {
      bf16x8 pw[2];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float e0 = live ? __builtin_amdgcn_exp2f(z[u] - m2) : 0.f;
        const float e1 = live ? __builtin_amdgcn_exp2f(z[8 + u] - m2) : 0.f;
        l += e0 + e1;
        pw[0][u] = (__bf16)e0;
        pw[1][u] = (__bf16)e1;
      }
      // head row 32 hq + c, k steps 2 par and 2 par + 1 (this tile's rows)
      uint8_t* prow = plds + (32 * hq + c) * kPStride64 + 64 * par + 16 * hh;
      *(bf16x8*)prow = pw[0];
      *(bf16x8*)(prow + 32) = pw[1];
    }
    __syncthreads();                               // every head's P of both tiles is in place
    bf16x8 pa[2][4];
    if constexpr (F8) {
      // P times the rows' value scales of this wave's dim tile (k step kk: tile kk / 2, k slot
      // 8 hh + u is its row 16 (kk % 2) + 8 (u / 4) + 4 hh + u % 4)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const uint8_t* st = tbuf(b0 + (kk >> 1)) + 640 + 4 * wave;
        float vs[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          vs[u] = *(const float*)(st + (16 * (kk & 1) + 8 * (u >> 2) + 4 * hh + (u & 3)) * kSfaRowF8);
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          const float* pr = (const float*)(plds + (32 * hb + c) * PS) + 16 * kk + 8 * hh;
          const f32x4 p0 = *(const f32x4*)pr, p1 = *(const f32x4*)(pr + 4);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            pa[hb][kk][u] = (__bf16)(p0[u] * vs[u]);
            pa[hb][kk][4 + u] = (__bf16)(p1[u] * vs[4 + u]);
          }
        }
      }
      const int tg = lane >> 4, tu = (lane & 15) >> 1;
      const int trow = 8 * (tu >> 2) + 4 * (tg >> 1) + (tu & 3);
      const int tdim = 128 * wave + 16 * (tg & 1) + 8 * (lane & 1);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        bf16x8 b[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const v2i32 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) v2i32*)(
              tbuf(b0 + (kk >> 1)) + (16 * (kk & 1) + trow) * kSfaRowF8 + 32 * nb + tdim));
          b[kk] = widen_fp8x8(u32x2{(uint32_t)v.x, (uint32_t)v.y}, 1.f);
        }
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
          for (int kk = 0; kk < 4; ++kk)
            o[hb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[hb][kk], b[kk], o[hb][nb], 0, 0, 0);
      }
      tc.computed();
      continue;
    }
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        pa[hb][kk] = *(const bf16x8*)(plds + (32 * hb + c) * kPStride64 + 32 * kk + 16 * hh);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int dim = 128 * wave + 32 * nb + vdim;
      const int cho = tile_off(0, dim >> 3) + 2 * (dim & 7);
      bf16x8 b[4];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        s16x4 v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          v[q] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4*)(tbuf(b0 + tt) + tile_off(8 * q + vrow, 0) + cho));
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
          b[2 * tt + kk] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v[2 * kk], v[2 * kk + 1], 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          o[hb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[hb][kk], b[kk], o[hb][nb], 0, 0, 0);
    }
    tc.computed();
  }

  tl_stamp(p.tl, kTlSfa, kTlLoopDone);
  tl_clock(p.tl, kTlSfa, kTlClockEnd);
  tc.put(p.tl, kTlSfa, npairs);
  // per-head totals over the two tiles of each pair; flags of both waves of a head half
  const float lw = xhalf_sum(l);
  const uint32_t ow = (uint32_t)__ballot(over);
  if (hh == 0) xsum[wave][c] = lw;
  if (lane == 0) xover[wave] = ow;
  __syncthreads();
  const float lt = lw + xsum[wave ^ 2][c];
  const uint32_t flagword = ow | xover[wave ^ 2];
  if (par == 0 && hh == 0) hv[32 * hq + c] = lt > 0.f ? 1.f / lt : 0.f;
  __syncthreads();
  const int hgb = hg * 64;                         // first head of the workgroup
  // accumulator (hb, nb) element 4j + i of lane (hh, c): head hgb + 32hb + 8j + 4hh + i,
  // dim 128 wave + 32 nb + c
  if (p.nsplit == 1) {
    uint16_t* out = (uint16_t*)p.out + ((size_t)t * p.H + hgb) * kSfaDv + 128 * wave + c;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 inv = *(const f32x4*)&hv[32 * hb + 8 * j + 4 * hh];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int hd = 32 * hb + 8 * j + 4 * hh + i;
#pragma unroll
          for (int nb = 0; nb < 4; ++nb)
            out[hd * kSfaDv + 32 * nb] = __builtin_bit_cast(uint16_t, (__bf16)(o[hb][nb][4 * j + i] * inv[i]));
        }
      }
    if (p.lse && par == 0 && hh == 0)
      p.lse[(size_t)t * p.H + h0 + c] = lt > 0.f ? (m2 + log2f(lt)) * kLn2 : -INFINITY;
  } else {
    // O / l of this slice in fp16, records as the accumulators lie in the registers: record
    // (hb*4 + j)*2 + np of lane (hh, c) holds heads 32hb + 8j + 4hh + i (i < 4) at dims
    // 128 wave + 32(2np + s) + c (s < 2), value 4s + i; 16 KB per (query, head group, slice,
    // wave)
    // (slices of one record adjacent, as in the 128-head kernel: 16 records per wave)
    uint8_t* po = (uint8_t*)p.part_o +
                  ((((size_t)t * p.n_hg + hg) * NW + wave) * 16 * p.nsplit + r) * 1024 + 16 * lane;
    // streaming stores with up to 16 slices (measured: 128K decode, 16 slices, attention 27.7
    // -> 27.0 us; one 1M query, 64 slices of one tile, 24.7 -> 25.4 us with them)
    const bool nt = p.nsplit <= 16;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 inv = *(const f32x4*)&hv[32 * hb + 8 * j + 4 * hh];
#pragma unroll
        for (int np = 0; np < 2; ++np) {
          uint32_t w[4];
#pragma unroll
          for (int sd = 0; sd < 2; ++sd)
#pragma unroll
            for (int i = 0; i < 4; i += 2) {
              const _Float16 a = (_Float16)(o[hb][2 * np + sd][4 * j + i] * inv[i]);
              const _Float16 b = (_Float16)(o[hb][2 * np + sd][4 * j + i + 1] * inv[i + 1]);
              w[2 * sd + i / 2] = (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
            }
          u32x4* dst = (u32x4*)(po + (size_t)((hb * 4 + j) * 2 + np) * p.nsplit * 1024);
          if (nt) __builtin_nontemporal_store(u32x4{w[0], w[1], w[2], w[3]}, dst);
          else *dst = u32x4{w[0], w[1], w[2], w[3]};
        }
      }
    if (par == 0 && hh == 0) {
      float* pm = p.part_ml + (((size_t)t * p.H + h0 + c) * p.nsplit + r) * 2;
      pm[0] = m2;
      pm[1] = lt;
    }
  }
  tl_stamp(p.tl, kTlSfa, kTlWritten);
  if (par == 0 && lane == 0) p.flags[((size_t)t * (p.H / 32) + hg * 2 + hq) * p.nsplit + r] = flagword;
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
  const bool f8 = p.kv_dtype == kDtFP8;
  auto kvat = [&](int64_t row, int d) -> float {
    if (f8) {
      const uint8_t* r8 = (const uint8_t*)p.kv + (size_t)row * kSfaRowF8;
      if (d < kSfaDv) return fp8_e4m3_to_f32(r8[d]) * ((const float*)(r8 + 640))[d >> 7];
      return bf16_bits_to_f32(((const uint16_t*)(r8 + kSfaDv))[d - kSfaDv]);
    }
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

// Merge of the index-list slices.  A workgroup owns (query, 16 heads of one 32-head block, the
// output dims of one wave of the MFMA kernel): the log-sum-exp weights of the slices, then per
// thread one 16-byte record of the fp16 partials per slice, summed in fp32.  Heads flagged by
// the MFMA kernel (scores far above the exponent reference) are recomputed by the reference
// method in the workgroup of the first dim range and skipped by the others; a head whose
// merged output is not finite (a partial beyond the fp16 range) is recomputed by the
// workgroup that saw it.  With a single slice the MFMA kernel wrote the output and only the
// flags are checked.
constexpr int kCombineThreads = 256;
constexpr int kMaxSlices = 64;
static_assert(kMaxTopK / kTileRows <= kMaxSlices, "a slice holds at least one tile");
// partial loads in flight per thread: the combine kernel is built for batches of 8, 16 and 32
// slices and launched with the smallest that covers the slices in one batch (a batch's
// records take 4 VGPRs each, and a larger batch than needed costs registers: at 32 the kernel
// runs one workgroup per SIMD and moves the first loads' results through AGPRs, which makes
// the compiler wait for them before the rest of the batch is issued)

__device__ __forceinline__ float wave_max(float v) {
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

template <int kCombineBatch>
__global__ __launch_bounds__(kCombineThreads) void sfa_combine_kernel(SfaParams p) {
  __shared__ RefSmem ws;
  __shared__ __attribute__((aligned(16))) float wgt[kMaxSlices][16];
  __shared__ uint32_t flagged, nonfinite;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int HB = p.heads_per_wg / 32;                 // 32-head blocks of an attention workgroup
  const int DWV = p.dim_waves;                        // its waves, each owning DW output dims
  const int DW = kSfaDv / DWV, NB = DW / 32;
  const int half = blockIdx.x & 1;
  const int hb = (blockIdx.x >> 1) % HB;
  const int w = (blockIdx.x >> 1) / HB % DWV;
  const int hg = (blockIdx.x >> 1) / (HB * DWV);
  const int t = blockIdx.y;
  const int hw = hg * HB + hb;                        // 32-head block
  const int hb0 = hw * 32 + 16 * half;                // heads hb0 .. hb0 + 15
  const int S = p.nsplit;
  tl_stamp(p.tl, kTlCombine, kTlStart);
  const int nslot = NB * 64;
  const int nrec = HB * 4 * (NB / 2);                 // records of one attention wave
  const uint8_t* blk = (const uint8_t*)p.part_o + (((size_t)t * p.n_hg + hg) * DWV + w) * nrec * S * 1024;
  const size_t rstride = 1024;                        // from one slice to the next
  // the slices' flag words of this 32-head block (wave 0, lane r: slice r), reduced once the
  // other loads are in flight
  // (loads from clamped addresses, masked at use: a load under a lane condition made the
  // compiler wait for it in place)
  const int sl = min(lane, S - 1);
  uint32_t fl = 0u;
  if (wave == 0) fl = p.flags[((size_t)t * (p.H / 32) + hw) * S + sl];
  // slot (record, lane) of this thread: record (hb*4 + j)*(NB/2) + np with j = 2*half + jl,
  // value 4s + i: head hb0 + 8jl + 4hh + i, dim DW*w + 32(2np + s) + c
  auto src_of = [&](int slot) {
    const int ln = slot & 63, rl = slot >> 6;
    const int rec = (hb * 4 + 2 * half + rl / (NB / 2)) * (NB / 2) + rl % (NB / 2);
    return blk + (size_t)rec * S * 1024 + 16 * ln;
  };
  // Every load of the first batch is issued before any is used: the flags, the (m, l) pairs,
  // then this thread's records of the first kCombineBatch slices of its first slot, so that
  // the weights are computed while the partials are in flight and a combine of up to
  // kCombineBatch slices costs one memory round trip.
  u32x4 v0[kCombineBatch];
  if (S > 1) {
    // weights of heads 4*wave .. 4*wave + 3 (of the 16), lane r holding slice r
    float2 a[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      a[k] = *(const float2*)(p.part_ml + (((size_t)t * p.H + hb0 + 4 * wave + k) * S + sl) * 2);
    const uint8_t* src = src_of(tid);
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u)
      v0[u] = u < S ? *(const u32x4*)(src + (size_t)u * rstride) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float mk = lane < S ? a[k].x : -INFINITY;
      const float M = wave_max(mk);
      const float e = (M == -INFINITY || lane >= S) ? 0.f : exp2f(mk - M) * a[k].y;
      const float Lsum = wave_sum(e);
      if (lane < S) wgt[lane][4 * wave + k] = Lsum > 0.f ? e / Lsum : 0.f;
      if (p.lse && w == 0 && lane == 0)
        p.lse[(size_t)t * p.H + hb0 + 4 * wave + k] = Lsum > 0.f ? (M + log2f(Lsum)) * kLn2 : -INFINITY;
    }
  }
  if (wave == 0) {
    fl = lane < S ? fl : 0u;
    for (int off = 32; off >= 1; off >>= 1) fl |= (uint32_t)__shfl_xor((int)fl, off, 64);
    if (lane == 0) {
      flagged = (fl >> (16 * half)) & 0xffffu;
      nonfinite = 0u;
    }
  }
  __syncthreads();
  if (S > 1) {
    for (int slot = tid; slot < nslot; slot += kCombineThreads) {
      const int ln = slot & 63, jl = (slot >> 6) / (NB / 2), np = (slot >> 6) % (NB / 2);
      const int hh = ln >> 5, c = ln & 31;
      const uint8_t* src = src_of(slot);
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      auto accumulate = [&](const u32x4 (&v)[kCombineBatch], int r0) {
#pragma unroll
        for (int u = 0; u < kCombineBatch; ++u) {
          const f32x4 wr = r0 + u < S ? *(const f32x4*)&wgt[r0 + u][8 * jl + 4 * hh] : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t bits = (v[u][e >> 1] >> (16 * (e & 1))) & 0xffffu;
            acc[e] += wr[e & 3] * (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
          }
        }
      };
      for (int r0 = 0; r0 < S; r0 += kCombineBatch) {
        // the first batch of the first slot was loaded before the weights
        if (slot != (int)tid || r0 != 0) {
#pragma unroll
          for (int u = 0; u < kCombineBatch; ++u)
            v0[u] = r0 + u < S ? *(const u32x4*)(src + (size_t)(r0 + u) * rstride) : u32x4{0u, 0u, 0u, 0u};
        }
        accumulate(v0, r0);
      }
      const uint32_t skip = flagged >> (8 * jl + 4 * hh);
      uint16_t* out = (uint16_t*)p.out + ((size_t)t * p.H + hb0 + 8 * jl + 4 * hh) * kSfaDv + DW * w + 64 * np + c;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = e & 3, sd = e >> 2;
        if ((skip >> i) & 1u) continue;
        if (!__builtin_isfinite(acc[e])) atomicOr(&nonfinite, 1u << (8 * jl + 4 * hh + i));
        out[i * kSfaDv + 32 * sd] = (uint16_t)f32_to_bf16_bits(acc[e]);
      }
    }
  }
  __syncthreads();
  tl_stamp(p.tl, kTlCombine, kTlWritten);
  uint32_t mm = (w == 0 ? flagged : 0u) | nonfinite;
  while (mm) {
    const int k = __builtin_ctz(mm);
    mm &= mm - 1;
    reference_head<kCombineThreads>(p, t, hb0 + k, ws);
    __syncthreads();
  }
}

// With a single slice the MFMA kernel wrote the output itself; this kernel only looks at the
// flags (one word per 32 heads of a query, one per thread) and recomputes every flagged head
// by the reference method, one after the other in the workgroup that found it.
__global__ __launch_bounds__(kCombineThreads) void sfa_flag_fixup_kernel(SfaParams p) {
  __shared__ RefSmem ws;
  __shared__ uint32_t found[kCombineThreads];
  __shared__ int nfound;
  const int n_hw = p.H / 32;
  const int wid = blockIdx.x * kCombineThreads + threadIdx.x;   // (query, 32-head block)
  if (threadIdx.x == 0) nfound = 0;
  __syncthreads();
  if (wid < p.T * n_hw) {
    const uint32_t f = p.flags[wid];
    if (f) found[atomicAdd(&nfound, 1)] = (uint32_t)wid;
  }
  __syncthreads();
  const int nf = nfound;
  for (int q = 0; q < nf; ++q) {
    const uint32_t w = found[q];
    const int t = (int)(w / n_hw), hw = (int)(w % n_hw);
    uint32_t m = p.flags[w];
    while (m) {
      const int k = __builtin_ctz(m);
      m &= m - 1;
      reference_head<kCombineThreads>(p, t, hw * 32 + k, ws);
      __syncthreads();
    }
  }
}

}  // namespace

SfaPlan plan_sfa(int32_t T, int32_t H, int32_t K, int32_t dv, bool fast_path, bool kv_fp8) {
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
    pl.heads_per_wg = (H % 128 == 0) ? 128 : (H % 64 == 0) ? 64 : 32;
    // Small decode batches take the 64-head variant (bf16 or fp8 rows).  A workgroup of either
    // kind reads its heads' queries plus its slice's rows: with at most 16 queries' worth of
    // 128-head groups the 128-head slices hold at most 128 rows, fewer bytes than the 147 KB
    // of queries, and halving the heads while doubling the rows reads the same bytes and
    // writes half the partial outputs; with more queries the rows dominate and the 128-head
    // workgroup reads less.
    pl.decode64 = !wide && H % 64 == 0 && (int64_t)T * (H / 64) <= 32;
    if (pl.decode64) pl.heads_per_wg = 64;
    if (const int v = plan_overrides().sfa_hpw; (v == 32 || v == 64 || v == 128) && H % v == 0) {
      pl.heads_per_wg = v;
      pl.decode64 = v == 64;
    }
    pl.n_hg = H / pl.heads_per_wg;
    pl.dim_waves = pl.decode64 ? 4 : pl.heads_per_wg / 32;
    const int64_t max_ns = (K + kTileRows - 1) / kTileRows;
    int64_t ns = 1;
    if (!wide) {
      const int64_t want = 256;
      ns = (want + (int64_t)T * pl.n_hg - 1) / ((int64_t)T * pl.n_hg);
      if (plan_overrides().sfa_splits > 0) ns = plan_overrides().sfa_splits;
      // slices of at most 1024 rows (kRows64 = 512 for the 64-head variant)
      const int64_t cap = pl.decode64 ? kRows64 : 1024;
      const int64_t min_ns = (K + cap - 1) / cap;
      if (ns < min_ns) ns = min_ns;
    }
    if (ns > max_ns) ns = max_ns;
    int64_t rps = (K + ns - 1) / ns;
    rps = (rps + kTileRows - 1) / kTileRows * kTileRows;
    pl.rows_per_split = (int32_t)rps;
    pl.nsplit = (int32_t)((K + rps - 1) / rps);
  }
  size_t off = 0;
  pl.off_zero = off;                     // never written: stays as the caller zeroed it
  off = al(off + 16);
  pl.off_flags = off;
  off = al(off + (size_t)T * ((H + 31) / 32) * pl.nsplit * 4);
  pl.off_part = off;
  if (pl.nsplit > 1) off = al(off + (size_t)T * H * pl.nsplit * dv * 2);
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
  const bool f8 = p.kv_dtype == kDtFP8;
  if (p.decode64) {
    if (f8) hipLaunchKernelGGL(sfa_mfma64_kernel<true>, grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL(sfa_mfma64_kernel<false>, grid, dim3(256), 0, stream, p);
  } else switch (p.heads_per_wg) {
    case 128:
      if (f8) hipLaunchKernelGGL((sfa_mfma_kernel<4, true>), grid, dim3(256), 0, stream, p);
      else hipLaunchKernelGGL((sfa_mfma_kernel<4, false>), grid, dim3(256), 0, stream, p);
      break;
    case 64:
      if (f8) hipLaunchKernelGGL((sfa_mfma_kernel<2, true>), grid, dim3(128), 0, stream, p);
      else hipLaunchKernelGGL((sfa_mfma_kernel<2, false>), grid, dim3(128), 0, stream, p);
      break;
    default:
      if (f8) hipLaunchKernelGGL((sfa_mfma_kernel<1, true>), grid, dim3(64), 0, stream, p);
      else hipLaunchKernelGGL((sfa_mfma_kernel<1, false>), grid, dim3(64), 0, stream, p);
      break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // merges the slices, and recomputes any flagged head (with one slice it only checks flags)
  if (p.nsplit > 1) {
    const int hb = p.heads_per_wg / 32;
    const dim3 cg(p.n_hg * hb * p.dim_waves * 2, p.T);
    if (p.nsplit <= 8) hipLaunchKernelGGL(sfa_combine_kernel<8>, cg, dim3(kCombineThreads), 0, stream, p);
    else if (p.nsplit <= 16) hipLaunchKernelGGL(sfa_combine_kernel<16>, cg, dim3(kCombineThreads), 0, stream, p);
    else hipLaunchKernelGGL(sfa_combine_kernel<32>, cg, dim3(kCombineThreads), 0, stream, p);
  } else {
    const int words = p.T * (p.H / 32);
    hipLaunchKernelGGL(sfa_flag_fixup_kernel, dim3((words + kCombineThreads - 1) / kCombineThreads),
                       dim3(kCombineThreads), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace dsa
