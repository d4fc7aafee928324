// Lightning indexer fused with exact Top-K (gfx950).
//
// What it computes: for query t of sequence b, visible prefix V, and each position s < V,
//   S[s] = sum_h w[t,h] * ReLU(q[t,h,:] . key(s))
// then the K_eff = min(K, V) best positions (score descending, lower position first).
// Scoring, head-weighted aggregation and Top-K run in one kernel that reads the paged key
// cache directly and writes only the index list: the fused index operator of "Large Model
// Inference Acceleration: Day-0 Adaptation..." (section 1.1) and of "Day0 Adaptation and
// Sparse Attention Optimization for Long-Sequence LLM Inference" (section 4).  The per-head
// scores never leave the registers and the per-position scores stay in LDS.
//
// Work decomposition (MI355X: 256 CUs in 8 XCDs, wave64, 160 KB LDS per CU):
//   * one workgroup of 4 waves per (query, context split of `split` positions), two per CU.
//     With the host's total of the visible lengths and at most 64 queries the splits are
//     sized so that the live items fit the resident slots and the grid numbers only live
//     items; with many queries and bf16 or fp8 keys (chunked prefill) a workgroup takes four
//     queries of one sequence over one split instead (see score_mq);
//   * scoring: each wave takes a contiguous run of 32-position groups.  Key bytes travel
//     HBM -> LDS with fully coalesced direct-to-LDS loads into a per-wave ring of groups.  Per
//     group, one v_mfma_f32_32x32x16_bf16 chain per 32-head half computes x[head, position]
//     (keys as the B operand, read back from LDS in MFMA lane layout; fp8 keys widened to
//     bf16 exactly), then each lane applies ReLU and the head weights to the 16 accumulator
//     rows it holds and one cross-lane add finishes the head sum.  The fp8 per-token scale
//     multiplies the head sum (ReLU(c x) = c ReLU(x) for c > 0).  Every position goes
//     through the same instruction sequence, so bit-identical keys get bit-identical scores
//     wherever they sit;
//   * each split picks a threshold key by radix selection over its LDS scores so that a
//     little more than its expected share of the Top-K survives, and writes those candidates
//     (order-preserving key, position) in position order to its own run of the workspace;
//   * the last split of a query to arrive (atomic counter) copies the runs into LDS in split
//     order, finds the exact K_eff-th key by radix selection, and checks that every split's
//     threshold lies at or below it - then the candidates provably contain the exact answer.
//     A split whose threshold was too high is re-scored by the merging workgroup and
//     contributes its exact local Top-K instead (rare unless the top positions crowd into a
//     few splits; always correct).
//   * Cross-workgroup data (candidates, split headers, the arrival counter) is written and read
//     only with agent-scope atomic operations (relaxed loads, stores and increments), which are
//     coherent across the XCDs' separate L2 caches without writing back or invalidating those
//     caches, so no two workgroups' accesses form a data race.  The hand-off's order comes from
//     completion: every writer waits until its stores have completed before the increment, and
//     the last arriver issues its loads only after its increment has returned.  Release and
//     acquire fences at agent scope would state that order in the memory model, but on gfx950
//     they write back and invalidate the L2 at every arrival (measured: 43.4 -> 46.0 us on
//     eight 64K-128K queries, 69.4 -> 82.4 us on 32 x 32K).
// Code that runs once per workgroup is kept in loops rather than unrolled: it executes cold
// from the instruction cache, so its size, not its instruction count, sets its time.
// A query whose prefix fits one split does the exact selection in place.
// A reference path (any supported dtypes and head geometry) scores each position in fp64.

#include <cstdlib>

#include "dsa_internal.hpp"

namespace dsa {
namespace {

constexpr int NT = kIdxThreads;
constexpr int NWAVE = NT / 64;
constexpr int kBins = 2048;               // radix bins per pass

// LDS ring of the MFMA scorer: D slots per wave (D a power of two), each holding one
// 32-position group of keys (+ its fp8 scales).
template <int MODE> struct Ring { static constexpr int D = 1, SLOT = 0; };
template <> struct Ring<1> { static constexpr int D = 2, SLOT = 8192; };          // bf16 keys
template <> struct Ring<2> { static constexpr int D = 4, SLOT = 4096 + 256; };    // fp8 keys + scales
template <> struct Ring<3> : Ring<2> {};
constexpr int kMqQ = 4;        // queries of a multi-query workgroup (one per wave)
constexpr int kMqRing = 4;     // its shared ring of 8 KB bf16 key groups
// Where a multi-query workgroup keeps things in the shared region while it scores: the
// histogram the split selection uses stays at its start, the scores of queries 1.. follow
// (query 0's are in the key array), and the ring takes the upper half.
constexpr int kMqKeysOff = kBins * 4;
constexpr int kMqRingOff = 32768;
constexpr int kMqMinT = 256;   // fewest queries for multi-query workgroups                                           // MXFP8 keys + scale bytes

// Bytes of the kernel's shared region: the scorer's ring while scoring, then the selection
// arrays.
template <int MODE>
constexpr int region_bytes() {
  return MODE == 0 ? 65536 : Ring<MODE>::D * NWAVE * Ring<MODE>::SLOT;
}
// Merge layout of the region: the run starts of the query's splits at its end; the candidate
// runs copied in split order (keys, then positions) from its start when the selection runs on
// that list alone (merge_fast), else after a selection area (keys, then virtual indices turned
// positions) that the general merge uses.
constexpr int kSelCap = kMaxTopK + 64;           // the selection and one histogram bin
constexpr int kSelBytes = kSelCap * 8;
template <int MODE>
constexpr int flat_words() {
  return (region_bytes<MODE>() - kSelBytes) / 4;
}

// Pointers to the kernel's LDS arrays.
struct Lds {
  uint32_t* keys;     // [kSplitMax] order-preserving score keys of the split
  const float* w;     // [NWAVE][64] head weights, one copy per wave (MFMA paths)
  uint8_t* region;    // region_bytes<MODE>()
  int* hist;          // [kBins]
  uint32_t* sel_key;  // [kSelCap] merge: keys of the selection (and a few more)
  int32_t* sel_pos;   // [kSelCap] merge: their positions
  uint32_t* flat;     // [flat_words] merge: run starts, candidate keys (+ positions)
  int* res;           // [4]
  int* scan;          // [2 * NWAVE + 2]
  int* wcnt;          // [2 * NWAVE]
  int* bcast;         // [4]
  uint32_t* range;    // [2 * NWAVE] per-wave smallest and largest score key of the split
  int* psum;          // [NT] partial histogram sums
  uint32_t* small;    // [64] keys of one histogram bin
  uint32_t* small_w;  // [64] merge: the wave that gathered each of them
};

struct GenericSmem {
  float q[kGenericMaxHD];
  float w[kGenericMaxHeads];
};

// cross-workgroup stores and loads (see the header comment)
__device__ __forceinline__ void st_agent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_agent(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t ld_agent(const int32_t* p) {
  return __hip_atomic_load(const_cast<int32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until every memory operation this wave issued has completed.
__device__ __forceinline__ void wait_all_memory() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt((N & 0xf) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

typedef __attribute__((address_space(4))) const int32_t const_i32;

// LDS byte address of a pointer into LDS.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Direct-to-LDS load: each active lane l reads SIZE bytes (16 or 4) at gbase + voff and they
// land at LDS byte address lds + SIZE * l; gbase and lds are wave-uniform.  AGENT makes it an
// agent-scope (cross-XCD coherent) read, like ld_agent.  Issued as inline asm, so the
// compiler does not see these LDS writes (its own wait insertion would otherwise drain every
// outstanding load before each LDS read); the callers wait for them with vmcnt, and the asm's
// memory clobber keeps the compiler from moving LDS accesses across it.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <int SIZE, bool AGENT = false>
__device__ __forceinline__ void load_to_lds(const void* gptr, uint32_t voff, uint32_t lds_in) {
  static_assert(SIZE == 16 || SIZE == 4, "load size");
  // the operands are wave-uniform; make them scalar for the instruction's SGPR fields
  const uint64_t ga = (uint64_t)(uintptr_t)gptr;
  const uint32_t glo = __builtin_amdgcn_readfirstlane((uint32_t)ga);
  const uint32_t ghi = __builtin_amdgcn_readfirstlane((uint32_t)(ga >> 32));
  const void* gbase = (const void*)(uintptr_t)(((uint64_t)ghi << 32) | glo);
  const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_in);
  if constexpr (SIZE == 16 && AGENT)
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 sc1"
                 :: "v"(voff), "s"(gbase), "s"(lds) : "memory", "m0");
  else if constexpr (SIZE == 16)
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(voff), "s"(gbase), "s"(lds) : "memory", "m0");
  else if constexpr (AGENT)
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1 sc1"
                 :: "v"(voff), "s"(gbase), "s"(lds) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
                 :: "v"(voff), "s"(gbase), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop

// ---------------------------------------------------------------------------------------
// Wave-level cross-lane operations on DPP (row shifts within 16-lane rows, then row
// broadcasts across them): a few VALU cycles per step instead of an LDS round trip.
// ---------------------------------------------------------------------------------------
template <class Op>
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, uint32_t id, Op op) {
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x111, 0xf, 0xf, false));  // row_shr:1
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x112, 0xf, 0xf, false));  // row_shr:2
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x114, 0xf, 0xf, false));  // row_shr:4
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x118, 0xf, 0xf, false));  // row_shr:8
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x142, 0xa, 0xf, false));  // row_bcast:15
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return v;
}
__device__ __forceinline__ int wave_scan_add(int v) {
  return (int)wave_incl_scan((uint32_t)v, 0u, [](uint32_t a, uint32_t b) { return a + b; });
}
__device__ __forceinline__ uint32_t wave_min(uint32_t v) {
  v = wave_incl_scan(v, 0xffffffffu, [](uint32_t a, uint32_t b) { return min(a, b); });
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  v = wave_incl_scan(v, 0u, [](uint32_t a, uint32_t b) { return max(a, b); });
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// ---------------------------------------------------------------------------------------
// Scoring
// ---------------------------------------------------------------------------------------

// max(x, 0) for any non-NaN float as one integer max on its bits: every negative float
// (and -0) has a negative int32 pattern and maps to +0; non-negative floats are unchanged.
__device__ __forceinline__ float relu(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

// MFMA scorer: q bf16 [64 heads x 128 dims], keys bf16 or fp8 (128 per token).
// Lane layout of v_mfma_f32_32x32x16_bf16: lane l supplies row/column (l & 31) and the
// 8-element k-slice 8*(l >> 5) .. +7; accumulator element r of lane l is
// D[8*(r/4) + 4*(l>>5) + (r%4)][l & 31].  The 128 key dims are assigned to k-slices so that
// lane half h takes dims [64h, 64h+64) of its key row; the query uses the same assignment,
// so every MFMA step still pairs equal dims.
// Key rows of a group land in the ring with coalesced direct-to-LDS loads (each load
// instruction moves 1 KB: whole 128-byte lines per 8 or 16 lanes); each row's 16-byte chunks
// are XOR-swizzled by the row index so that the MFMA-layout reads back from LDS hit distinct
// banks.  A group lies in one page (pages hold >= 32 tokens; splits start at multiples of
// 64), whose block id is one wave-uniform scalar load.  Group indices past the wave's run
// are clamped onto its last group (harmless re-reads) so every step issues the same loads
// and the hardware waits stay exact.
// MXFP8 keys (MODE 3) move like fp8 keys (128 code bytes and a 4-byte word of E8M0 scales per
// token); the codes are widened with their group's power-of-two scale, exactly, and the
// query is quantized to MXFP8 by the workgroup and dequantized into LDS (exact in bf16 for
// scale bytes >= 3, i.e. groups whose largest magnitude is at least 2^-116), so the products
// are the bf16 path's and every sum is the same fp32 accumulation.
template <bool FP8, bool PAGED, int MODE>
__device__ __forceinline__ void score_mfma(const IndexerParams& p, int t, int seq, int start,
                                           int len, const Lds& L, uint32_t& kr_lo, uint32_t& kr_hi) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5, col = lane & 31;
  constexpr int ROWB = FP8 ? 128 : 256;       // bytes per key row
  constexpr int CPR = ROWB / 16;              // 16-byte chunks per row
  constexpr int GB = 32 * ROWB;               // key bytes per group
  constexpr int NI = GB / 1024;               // direct-to-LDS loads per group (keys)
  constexpr int D = Ring<MODE>::D;            // ring depth: D-1 groups in flight
  constexpr int SLOT = Ring<MODE>::SLOT;
  constexpr int LPG = NI + (FP8 ? 1 : 0);     // loads per group
  constexpr int RPI = 1024 / ROWB;            // rows per load instruction
  constexpr int LPR = 64 / RPI;               // lanes per row in a load instruction
  static_assert(GB + (FP8 ? 256 : 0) <= SLOT, "slot size");
  static_assert((D & (D - 1)) == 0, "ring depth is a power of two");

  const int ngroups = (len + 31) >> 5;
  const int per = (ngroups + NWAVE - 1) / NWAVE;
  const int g0 = min(ngroups, wave * per), g1 = min(ngroups, g0 + per);
  constexpr bool MX = MODE == 3;
  // MXFP8 keys: the query was quantized once for the call (mx_query_kernel) and is read like
  // a bf16 query from its dequantized values
  const uint16_t* qb = (MX ? (const uint16_t*)p.q_mx : (const uint16_t*)p.q) + (size_t)t * (64 * 128);
  static_assert(kSplitMax / 32 / NWAVE <= 64, "one lane per group of a wave's run");
  // The query's 64 x 128 bf16 values (16 KB) land once per workgroup in the ring's last slots
  // (slot D - 1 of every wave, at least 16 KB, first filled by the loop's first step), with
  // the 16-byte chunk c of head row r at chunk c ^ (r & 15), so that the fragment reads below
  // (32 heads at one chunk) fall in distinct banks.  Four waves loading their fragments
  // straight from global memory would fetch each query four times per workgroup, about 32 MB
  // across a decode launch at its start.
  static_assert(NWAVE * SLOT >= 64 * 128 * 2, "the query fits in the ring's last slots");
  uint8_t* const qland = L.region + (D - 1) * (NWAVE * SLOT);
#pragma unroll
  for (int u = 0; u < 16 / NWAVE; ++u) {
    const int P = 64 * (wave + NWAVE * u) + lane;    // landing chunk: row P / 16, slot P % 16
    const int r = P >> 4;
    load_to_lds<16>(qb, (uint32_t)(r * 256 + 16 * ((P & 15) ^ (r & 15))),
                    lds_addr(qland + 1024 * (wave + NWAVE * u)));
  }
  // One round trip brings the query, this wave's copy of the head weights (LDS) and the
  // pages of its groups (lane l: the block id of group g0 + l).
  const float* lw = L.w + wave * 64;
  load_to_lds<4>(p.w + (size_t)t * 64, 4u * lane, lds_addr(lw));
  int gblk = 0;
  if constexpr (PAGED)
    gblk = p.L.bt[(int64_t)seq * p.L.bt_stride + ((start + 32 * max(0, min(g0 + lane, g1 - 1))) >> p.L.bs_log2)];
  wait_vmcnt<0>();
  __syncthreads();                            // every wave's share of the query has landed
  bf16x8 a0[8], a1[8];
  // head col and 32 + col share the swizzle (32 is a multiple of 16)
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int ch = (8 * half + s) ^ (col & 15);
    a0[s] = *(const bf16x8*)(qland + col * 256 + 16 * ch);
    a1[s] = *(const bf16x8*)(qland + (32 + col) * 256 + 16 * ch);
  }
  __syncthreads();                            // every wave holds its fragments: the ring may start
  if (g0 >= g1) return;
  uint32_t& kmin = kr_lo;
  uint32_t& kmax = kr_hi;
  const int bsl = PAGED ? p.L.bs_log2 : 0;
  const int64_t cbase = PAGED ? 0 : (int64_t)seq * p.L.seq_stride;
  const uint8_t* kbytes = (const uint8_t*)p.k_pool;
  const int cpos = lane % LPR;                // chunk position this lane fills in its row
  // slot k of this wave's ring
  uint8_t* const ring0 = L.region + wave * SLOT;
  auto slot_of = [&](int k) { return ring0 + k * (NWAVE * SLOT); };

  // Group g covers positions start + 32g + [0, 32) (the last group of a split stops at len;
  // its rows past the end re-read its last row).  All of them lie in one page, so the
  // group's first pool row is wave-uniform and the lanes add 32-bit offsets to it.
  auto issue = [&](int g, uint8_t* sb) {
    g = min(g, g1 - 1);
    const int gpos = start + 32 * g;
    const int last = len - 1 - 32 * g;        // last valid row of the group (>= 0)
    int64_t row0;
    if constexpr (PAGED) {
      const int blk = __builtin_amdgcn_readlane(gblk, g - g0);
      row0 = ((int64_t)blk << bsl) | (gpos & ((1 << bsl) - 1));
    }
    else row0 = cbase + gpos;
    const uint8_t* gbase = kbytes + row0 * ROWB;
    const uint32_t lb = lds_addr(sb);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = RPI * i + lane / LPR;
      const uint32_t off = (uint32_t)(min(r, last) * ROWB + 16 * (cpos ^ (r & (CPR - 1))));
      load_to_lds<16>(gbase, off, lb + 1024 * i);
    }
    if constexpr (FP8) load_to_lds<4>(p.k_scale + row0, 4u * (uint32_t)min(col, last), lb + GB);
  };
  // Group g's products: both 32-head chains of MFMAs over the key rows in slot sb.
  auto products = [&](const uint8_t* sb, f32x16& acc0, f32x16& acc1) {
    const uint8_t* rb = sb + col * ROWB;      // this lane's row
    // MXFP8: this lane's two groups 2 half, 2 half + 1 (k steps 0..3, 4..7)
    const uint32_t sw = MX ? *(const uint32_t*)(sb + GB + 4 * col) >> (16 * half) : 0u;
    const float xs0 = MX ? mx_scale_f32(sw & 255u) : 1.0f;
    const float xs1 = MX ? mx_scale_f32((sw >> 8) & 255u) : 1.0f;
    acc0 = f32x16{};
    acc1 = f32x16{};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      bf16x8 kb;
      if constexpr (FP8) {
        const float xs = s < 4 ? xs0 : xs1;
        const u32x4 v = *(const u32x4*)(rb + 16 * ((4 * half + (s >> 1)) ^ (col & (CPR - 1))));
        const uint32_t lo = (s & 1) ? v.z : v.x;
        const uint32_t hi = (s & 1) ? v.w : v.y;
        const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, xs, false);
        const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, xs, true);
        const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, xs, false);
        const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, xs, true);
        kb = bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
      } else {
        kb = *(const bf16x8*)(rb + 16 * ((8 * half + s) ^ (col & (CPR - 1))));
      }
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[s], kb, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[s], kb, acc1, 0, 0, 0);
    }
  };
  // Group g's scores from its products: ReLU, head weights, head sum, fp8 token scale.
  auto finish = [&](int g, const f32x16& acc0, const f32x16& acc1, float scale) {
    // head weights of accumulator rows 8*(r/4) + 4*half + (r%4): four consecutive floats;
    // four independent partial sums keep the dependent adds short
    float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const f32x4 w0 = *(const f32x4*)(lw + 8 * rg + 4 * half);
      const f32x4 w1 = *(const f32x4*)(lw + 32 + 8 * rg + 4 * half);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        part[u] = fmaf(w0[u], relu(acc0[4 * rg + u]), part[u]);
        part[u] = fmaf(w1[u], relu(acc1[4 * rg + u]), part[u]);
      }
    }
    const float psum = (part[0] + part[1]) + (part[2] + part[3]);
    float tot = psum + __shfl_xor(psum, 32, 64);
    if constexpr (FP8 && !MX) tot *= scale;
    const int off = g * 32 + col;
    if (half == 0 && off < len) {
      const uint32_t key = float_to_key(tot);
      L.keys[off] = key;
      kmin = min(kmin, key);
      kmax = max(kmax, key);
    }
  };

  // The query is in registers (the fragment reads above completed before the barrier), so
  // the only loads in flight in the loop are the ring's, and the loop's waits count them
  // exactly.  Only the split's own groups are loaded: at step g the groups g + 1 .. up to
  // g + D - 1 that exist are in flight, so nothing is left to drain after the last step.
  tl_stamp(p.tl, kTlIndexer, kTlLoopStart);
  for (int k = 0; k < D - 1 && g0 + k < g1; ++k) issue(g0 + k, slot_of(k));
  TlCycles tc;
#pragma unroll 1
  for (int g = g0; g < g1; ++g) {
    const int k = (g - g0) & (D - 1);
    const int ahead = g1 - 1 - g;              // groups after g
    tc.mark();
    if (ahead >= D - 1) {
      // refill the slot consumed in the previous step (its LDS reads have completed)
      issue(g + D - 1, slot_of((k + D - 1) & (D - 1)));
      wait_vmcnt<LPG * (D - 1)>();            // group g has landed in LDS
    } else if (D > 3 && ahead == 2) {
      wait_vmcnt<LPG * 2>();
    } else if (D > 2 && ahead == 1) {
      wait_vmcnt<LPG>();
    } else {
      wait_vmcnt<0>();
    }
    tc.waited();
    const uint8_t* sb = slot_of(k);
    f32x16 acc0, acc1;
    products(sb, acc0, acc1);
    // both chains are issued before any accumulator is read, so they interleave
    __builtin_amdgcn_sched_barrier(0);
    finish(g, acc0, acc1, FP8 && !MX ? *(const float*)(sb + GB + 4 * col) : 1.f);
    tc.computed();
  }
  tc.put(p.tl, kTlIndexer, g1 - g0);
}

// Multi-query scoring (bf16, fp8 or MXFP8 keys, kMqQ queries of one sequence over one split, as in a
// prefill chunk whose queries share the cached context).  Scoring one query per workgroup
// re-reads the split's keys for every query through a two-slot ring per wave, and is then
// bound by the latency of those loads.  Here the waves share one ring of kMqRing key groups
// (kMqRing - 1 in flight) filled once for all the queries: every wave issues two of a bf16
// group's eight direct-to-LDS loads (fp8: one of four, plus a copy of the group's 32 token
// scales, the same bytes from every wave), and one barrier per group makes the group visible
// to all waves and frees the slot of the previous one.  Wave w then scores query w with the same
// MFMA steps as score_mfma, into its own key array.  Waves without a query (nq < kMqQ) still
// load and pass the barriers.  Group indices past the split are clamped onto its last group,
// so that every step issues the same loads and the waits stay exact.  MXFP8 keys (MX) move
// like fp8 keys with their rows' scale bytes and are widened with their group's power-of-two
// scale; the queries were quantized to MXFP8 once for the call (mx_query_kernel).
template <bool FP8, bool PAGED, bool MX = false>
__device__ __forceinline__ void score_mq(const IndexerParams& p, const int (&tq)[kMqQ], int nq,
                                         int seq, int start, int lenmax, const int (&lens)[kMqQ],
                                         uint32_t* const (&keys)[kMqQ], const Lds& L,
                                         uint32_t* range) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5, col = lane & 31;
  constexpr int ROWB = FP8 ? 128 : 256;       // bytes per key row
  constexpr int CPR = ROWB / 16;              // 16-byte chunks per row
  constexpr int RPI = 1024 / ROWB;            // rows per load instruction
  constexpr int LPR = 64 / RPI;               // lanes per row in a load instruction
  constexpr int GB = 32 * ROWB;               // key bytes per group
  constexpr int KPW = GB / 1024 / NWAVE;      // key loads per wave and group
  constexpr int LPW = KPW + (FP8 ? 1 : 0);    // loads per wave and group
  constexpr int D = kMqRing, SLOT = 8192;
  static_assert(GB + (FP8 ? 256 : 0) <= SLOT && KPW >= 1, "slot size");
  static_assert(kMqRingOff + D * SLOT <= region_bytes<1>() &&
                kMqRingOff + D * SLOT <= region_bytes<2>() &&
                kMqRingOff + D * SLOT <= region_bytes<3>(), "ring size");
  static_assert(kMqKeysOff + (kMqQ - 1) * kSplitMax * 4 <= kMqRingOff, "scores below the ring");
  static_assert(kSplitMax / 32 <= 64, "one lane per group of the split");
  seq = __builtin_amdgcn_readfirstlane(seq);
  start = __builtin_amdgcn_readfirstlane(start);
  lenmax = __builtin_amdgcn_readfirstlane(lenmax);
  const int ng = (lenmax + 31) >> 5;
  const bool act = wave < nq;
  const int t = __builtin_amdgcn_readfirstlane(act ? tq[wave] : tq[0]);
  const int len = __builtin_amdgcn_readfirstlane(act ? lens[wave] : 0);
  uint32_t* const kout = keys[act ? wave : 0];

  // MXFP8 keys: the queries were quantized once for the call (mx_query_kernel) and are read
  // like bf16 queries from their dequantized values
  const uint16_t* qsrc = (MX ? (const uint16_t*)p.q_mx : (const uint16_t*)p.q) + (size_t)t * (64 * 128);
  bf16x8 a0[8], a1[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    a0[s] = *(const bf16x8*)(qsrc + col * 128 + half * 64 + 8 * s);
    a1[s] = *(const bf16x8*)(qsrc + (32 + col) * 128 + half * 64 + 8 * s);
  }
  const float* lw = L.w + wave * 64;
  load_to_lds<4>(p.w + (size_t)t * 64, 4u * lane, lds_addr(lw));
  int gblk = 0;
  if constexpr (PAGED)
    gblk = p.L.bt[(int64_t)seq * p.L.bt_stride + ((start + 32 * min(lane, ng - 1)) >> p.L.bs_log2)];
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  const int bsl = PAGED ? p.L.bs_log2 : 0;
  const int64_t cbase = PAGED ? 0 : (int64_t)seq * p.L.seq_stride;
  const uint8_t* kbytes = (const uint8_t*)p.k_pool;
  const int cpos = lane % LPR;
  auto slot_of = [&](int g) { return L.region + kMqRingOff + (g & (D - 1)) * SLOT; };
  auto issue = [&](int g) {
    uint8_t* sb = slot_of(g);
    g = min(g, ng - 1);
    const int gpos = start + 32 * g;
    const int last = lenmax - 1 - 32 * g;
    int64_t row0;
    if constexpr (PAGED) {
      const int blk = __builtin_amdgcn_readlane(gblk, g);
      row0 = ((int64_t)blk << bsl) | (gpos & ((1 << bsl) - 1));
    }
    else row0 = cbase + gpos;
    const uint8_t* gbase = kbytes + row0 * ROWB;
    const uint32_t lb = lds_addr(sb);
#pragma unroll
    for (int ii = 0; ii < KPW; ++ii) {
      const int i = KPW * wave + ii;
      const int r = RPI * i + lane / LPR;
      const uint32_t off = (uint32_t)(min(r, last) * ROWB + 16 * (cpos ^ (r & (CPR - 1))));
      load_to_lds<16>(gbase, off, lb + 1024 * i);
    }
    if constexpr (FP8) load_to_lds<4>(p.k_scale + row0, 4u * (uint32_t)min(col, last), lb + GB);
  };
  wait_vmcnt<0>();                            // query and head weights
  // The loop is software-pipelined: the MFMAs of group g + 1 are issued before the epilogue of
  // group g (ReLU, head weights, head sum, key), so that the matrix cores work on the next
  // group while the vector unit finishes this one (in order, a wave would otherwise idle
  // behind each dependent MFMA chain and then run its epilogue with the matrix cores idle).
  // The head weights stay in registers for the whole loop.  Only the split's own groups are
  // loaded: the waits count the groups still in flight behind the one awaited.
  static_assert(D == 4, "the waits below count up to two groups in flight");
  f32x4 wv[2][4];
#pragma unroll
  for (int rg = 0; rg < 4; ++rg) {
    wv[0][rg] = *(const f32x4*)(lw + 8 * rg + 4 * half);
    wv[1][rg] = *(const f32x4*)(lw + 32 + 8 * rg + 4 * half);
  }
  auto wait_behind = [&](int n) {             // n of this wave's later groups may be in flight
    if (n >= 2) wait_vmcnt<2 * LPW>();
    else if (n == 1) wait_vmcnt<LPW>();
    else wait_vmcnt<0>();
  };
  // group g's MFMAs into (acc0, acc1), and its fp8 token scale (read now: the slot is refilled
  // before the epilogue)
  auto products = [&](int g, f32x16& acc0, f32x16& acc1, float& tscale) {
    const uint8_t* sb = slot_of(g);
    const uint8_t* rb = sb + col * ROWB;
    // MXFP8: this lane's two groups 2 half, 2 half + 1 (k steps 0..3, 4..7)
    const uint32_t sw = MX ? *(const uint32_t*)(sb + GB + 4 * col) >> (16 * half) : 0u;
    const float xs0 = MX ? mx_scale_f32(sw & 255u) : 1.0f;
    const float xs1 = MX ? mx_scale_f32((sw >> 8) & 255u) : 1.0f;
    tscale = FP8 && !MX ? *(const float*)(sb + GB + 4 * col) : 1.f;
    acc0 = f32x16{};
    acc1 = f32x16{};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      bf16x8 kb;
      if constexpr (FP8) {
        const float xs = s < 4 ? xs0 : xs1;
        const u32x4 v = *(const u32x4*)(rb + 16 * ((4 * half + (s >> 1)) ^ (col & (CPR - 1))));
        const uint32_t lo = (s & 1) ? v.z : v.x;
        const uint32_t hi = (s & 1) ? v.w : v.y;
        const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, xs, false);
        const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, xs, true);
        const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, xs, false);
        const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, xs, true);
        kb = bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
      } else {
        kb = *(const bf16x8*)(rb + 16 * ((8 * half + s) ^ (col & (CPR - 1))));
      }
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[s], kb, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[s], kb, acc1, 0, 0, 0);
    }
  };
  // the epilogue's arithmetic (no branch, so that it can interleave with the next group's
  // MFMAs) ...
  auto epi_value = [&](const f32x16& acc0, const f32x16& acc1, float tscale) {
    float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int rg = 0; rg < 4; ++rg)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        part[u] = fmaf(wv[0][rg][u], relu(acc0[4 * rg + u]), part[u]);
        part[u] = fmaf(wv[1][rg][u], relu(acc1[4 * rg + u]), part[u]);
      }
    const float psum = (part[0] + part[1]) + (part[2] + part[3]);
    float tot = psum + __shfl_xor(psum, 32, 64);
    if constexpr (FP8 && !MX) tot *= tscale;
    return tot;
  };
  // ... and its key store
  auto epi_store = [&](int g, float tot) {
    const int off = g * 32 + col;
    const uint32_t key = float_to_key(tot);
    const bool in = half == 0 && off < len;
    kmin = in ? min(kmin, key) : kmin;
    kmax = in ? max(kmax, key) : kmax;
    if (in) kout[off] = key;
  };
  // One step: group g + 1's operand reads and MFMAs (past the last group they read a stale
  // slot; those results are never used) interleaved with group g's epilogue arithmetic: per
  // k step one LDS read, two MFMAs and a share of the vector work.
  auto step = [&](int g, f32x16& n0, f32x16& n1, float& nts, const f32x16& c0, const f32x16& c1,
                  float cts) {
    products(g + 1, n0, n1, nts);
    const float tot = epi_value(c0, c1, cts);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);  // VALU
    }
    __builtin_amdgcn_sched_barrier(0);
    epi_store(g, tot);
  };
  for (int g = 0; g < D - 1 && g < ng; ++g) issue(g);
  TlCycles tc;
  f32x16 accA0, accA1, accB0, accB1;
  float tsA = 1.f, tsB = 1.f;
  wait_behind(min(D - 2, ng - 1));            // group 0
  __syncthreads();
  if (D - 1 < ng) issue(D - 1);
  if (act) products(0, accA0, accA1, tsA);
  // two steps per trip, so that the accumulator pairs alternate without copies
#pragma unroll 1
  for (int g = 0; g < ng; g += 2) {
    // step g: group g's MFMAs are in (accA); issue group g + 1's into (accB), then finish g
    tc.mark();
    const bool next1 = g + 1 < ng;
    if (next1) {
      wait_behind(min(D - 2, ng - 2 - g));    // group g + 1
      __syncthreads();                        // every wave's loads of g + 1 are in, g's slot is free
      if (g + D < ng) issue(g + D);
    }
    tc.waited();
    if (act) step(g, accB0, accB1, tsB, accA0, accA1, tsA);
    tc.computed();
    if (!next1) break;
    // step g + 1: group g + 1's MFMAs are in (accB); issue group g + 2's into (accA)
    tc.mark();
    const bool next2 = g + 2 < ng;
    if (next2) {
      wait_behind(min(D - 2, ng - 3 - g));    // group g + 2
      __syncthreads();
      if (g + 1 + D < ng) issue(g + 1 + D);
    }
    tc.waited();
    if (act) step(g + 1, accA0, accA1, tsA, accB0, accB1, tsB);
    tc.computed();
  }
  tc.put(p.tl, kTlIndexer, ng);
  wait_vmcnt<0>();                            // no load may still target the ring afterwards
  kmin = wave_min(kmin);
  kmax = wave_max(kmax);
  if (lane == 0) {
    range[2 * wave] = kmin;
    range[2 * wave + 1] = kmax;
  }
  __syncthreads();
}

__device__ __forceinline__ float load_elem(const void* base, int dt, int64_t i) {
  if (dt == kDtF32) return ((const float*)base)[i];
  if (dt == kDtBF16) return bf16_bits_to_f32(((const uint16_t*)base)[i]);
  return fp8_e4m3_to_f32(((const uint8_t*)base)[i]);
}
// Value of an MXFP8 key element: code times 2^(byte - 127) of its group of 32 (fp64, exact).
__device__ __forceinline__ double mx_key(const IndexerParams& p, int64_t row, int d) {
  const int e = (int)((const uint8_t*)p.k_scale)[row * (p.D / 32) + (d >> 5)] - 127;
  return ldexp((double)fp8_e4m3_to_f32(((const uint8_t*)p.k_pool)[row * p.D + d]), e);
}

// Reference scorer: one thread per position, fp64 accumulation (products of the stored
// operands are exact in fp64), rounded once to fp32.
__device__ __forceinline__ void score_generic(const IndexerParams& p, int seq, int start, int len,
                                              uint32_t* lkeys, const GenericSmem& gs,
                                              uint32_t& kmin, uint32_t& kmax) {
  const int H = p.H, D = p.D;
  for (int i = threadIdx.x; i < len; i += NT) {
    const int64_t row = pool_row(p.L, seq, start + i);
    const double ks = (p.k_dtype == kDtFP8) ? (double)p.k_scale[row] : 1.0;
    const bool mx = p.k_dtype == kDtMX;
    double S = 0.0;
    for (int h = 0; h < H; ++h) {
      double x = 0.0;
      for (int d = 0; d < D; ++d)
        x = fma((double)gs.q[h * D + d],
                mx ? mx_key(p, row, d) : (double)load_elem(p.k_pool, p.k_dtype, row * D + d) * ks, x);
      S = fma((double)gs.w[h], fmax(x, 0.0), S);
    }
    const uint32_t key = float_to_key((float)S);
    lkeys[i] = key;
    kmin = min(kmin, key);
    kmax = max(kmax, key);
  }
}

// Score positions [start, start+len) into L.keys; returns the smallest and largest key.
// Ends with a workgroup barrier.
template <int MODE>
__device__ __forceinline__ void score_split(const IndexerParams& p, int t, int seq, int start,
                                            int len, const Lds& L, const GenericSmem* gs,
                                            uint32_t& lo, uint32_t& hi) {
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  if constexpr (MODE == 0) {
    score_generic(p, seq, start, len, L.keys, *gs, kmin, kmax);
  } else {
    // wave-uniform values kept in scalar registers
    t = __builtin_amdgcn_readfirstlane(t);
    seq = __builtin_amdgcn_readfirstlane(seq);
    start = __builtin_amdgcn_readfirstlane(start);
    len = __builtin_amdgcn_readfirstlane(len);
    if (p.L.bt) score_mfma<MODE >= 2, true, MODE>(p, t, seq, start, len, L, kmin, kmax);
    else score_mfma<MODE >= 2, false, MODE>(p, t, seq, start, len, L, kmin, kmax);
  }
  kmin = wave_min(kmin);
  kmax = wave_max(kmax);
  if ((threadIdx.x & 63) == 0) {
    L.range[threadIdx.x >> 6] = kmin;
    L.range[NWAVE + (threadIdx.x >> 6)] = kmax;
  }
  __syncthreads();
  lo = 0xffffffffu;
  hi = 0u;
#pragma unroll
  for (int w = 0; w < NWAVE; ++w) {
    lo = min(lo, L.range[w]);
    hi = max(hi, L.range[NWAVE + w]);
  }
}

// ---------------------------------------------------------------------------------------
// Radix selection over order-preserving keys, with digits fitted to the keys' range.
// A pass counts the keys in [base, base + width] by the digit (key - base) >> sh, where sh
// is the smallest shift that maps the whole range onto kBins bins.  Fitting the range
// spreads a set of near-equal top scores over many bins instead of the few bins that the
// keys' leading bits would give them, so the LDS histogram atomics rarely collide.  Once the
// bin holding the wanted rank is known, its few keys are gathered and ranked directly.
// The keys are keys[0, n), in LDS or global memory.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ int range_shift(uint32_t width) {
  const int bits = width ? 32 - __clz((int)width) : 0;
  return max(0, bits - 11);
}

// Smallest and largest key over the workgroup.
__device__ __forceinline__ void key_range(const uint32_t* keys, int n, const Lds& L,
                                          uint32_t& lo, uint32_t& hi) {
  uint32_t mn = 0xffffffffu, mx = 0u;
  for (int i0 = threadIdx.x; i0 < n; i0 += 4 * NT) {
    uint32_t k[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) k[u] = keys[min(i0 + u * NT, n - 1)];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      mn = min(mn, k[u]);
      mx = max(mx, k[u]);
    }
  }
  mn = wave_min(mn);
  mx = wave_max(mx);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    L.range[wave] = mn;
    L.range[NWAVE + wave] = mx;
  }
  __syncthreads();
  lo = 0xffffffffu;
  hi = 0u;
#pragma unroll
  for (int w = 0; w < NWAVE; ++w) {
    lo = min(lo, L.range[w]);
    hi = max(hi, L.range[NWAVE + w]);
  }
}

// Bin of rank r (1-based, counted from the largest key) in a histogram over [base, base+width]
// with shift sh: fills the histogram, then finds bin d with above(d) < r <= above(d) +
// hist[d], where above(d) counts the keys in bins above d.  Every wave finds the same
// result, so no barrier is needed to share it.
struct BinPick { int d, above, c; };
__device__ __forceinline__ BinPick find_in_hist(int r, const Lds& L);
__device__ __forceinline__ BinPick rank_bin(const uint32_t* keys, int n, uint32_t base,
                                            uint32_t width, int sh, int r, const Lds& L) {
  int* hist = L.hist;
  __syncthreads();   // earlier readers of the histogram are done
  for (int i = threadIdx.x; i < kBins; i += NT) hist[i] = 0;
  __syncthreads();
  for (int i0 = threadIdx.x; i0 < n; i0 += 4 * NT) {
    uint32_t o[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) o[u] = keys[min(i0 + u * NT, n - 1)] - base;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i0 + u * NT < n && o[u] <= width) atomicAdd(&hist[o[u] >> sh], 1);
  }
  __syncthreads();
  return find_in_hist(r, L);
}

// Bin of rank r in the filled histogram L.hist (see rank_bin).  Starts and ends with
// workgroup-wide steps only where noted: one barrier after the partial sums.
__device__ __forceinline__ BinPick find_in_hist(int r, const Lds& L) {
  const int* hist = L.hist;
  int* psum = L.psum;
  {
    // thread i: the sum of bins [8i, 8i + 8)
    const int4 v0 = *(const int4*)(hist + 8 * threadIdx.x);
    const int4 v1 = *(const int4*)(hist + 8 * threadIdx.x + 4);
    psum[threadIdx.x] = v0.x + v0.y + v0.z + v0.w + v1.x + v1.y + v1.z + v1.w;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  // level 1: lane l holds 32-bin group 63 - l (descending)
  const int4 q = *(const int4*)(psum + 4 * (63 - lane));
  const int c1 = q.x + q.y + q.z + q.w;
  const int s1 = wave_scan_add(c1);
  const uint64_t b1 = __ballot(s1 >= r);
  const int l1 = b1 ? __builtin_ctzll(b1) : 63;
  const int grp = 63 - l1;
  const int above1 = __builtin_amdgcn_readlane(s1 - c1, l1);
  // level 2: lane l < 32 holds bin 32*grp + 31 - l
  const int c2 = lane < 32 ? hist[32 * grp + 31 - lane] : 0;
  const int s2 = wave_scan_add(c2);
  const uint64_t b2 = __ballot(s2 >= r - above1);
  const int l2 = b2 ? __builtin_ctzll(b2) : 31;
  BinPick bp;
  bp.d = 32 * grp + 31 - l2;
  bp.above = above1 + __builtin_amdgcn_readlane(s2 - c2, l2);
  bp.c = __builtin_amdgcn_readlane(c2, l2);
  return bp;
}

// The k-th largest key T (1 <= k <= n), the number of keys above it (gt) and the number at
// or above it (ge); every key lies in [lo, hi].
struct Kth { uint32_t T; int gt, ge; };
__device__ __forceinline__ Kth radix_kth(const uint32_t* keys, int n, int k, uint32_t lo,
                                         uint32_t hi, const Lds& L) {
  uint32_t base = lo, width = hi - lo;
  int above = 0;
  for (;;) {
    const int sh = range_shift(width);
    const BinPick bp = rank_bin(keys, n, base, width, sh, k - above, L);
    base += (uint32_t)bp.d << sh;
    if (sh == 0) return Kth{base, above + bp.above, above + bp.above + bp.c};
    width = (1u << sh) - 1u;
    if (bp.c <= 64) {
      // gather the c keys of the bin and rank them within one wave
      uint32_t* small = L.small;
      if (threadIdx.x == 0) L.bcast[3] = 0;
      __syncthreads();
      for (int i0 = threadIdx.x; i0 < n; i0 += 4 * NT) {
        uint32_t kk[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) kk[u] = keys[min(i0 + u * NT, n - 1)];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const bool in = i0 + u * NT < n && kk[u] - base <= width;
          const uint64_t bl = __ballot(in);
          if (bl) {
            int at = 0;
            if ((threadIdx.x & 63) == 0) at = atomicAdd(&L.bcast[3], __popcll(bl));
            at = __builtin_amdgcn_readfirstlane(at);
            if (in) small[at + __popcll(bl & ((1ull << (threadIdx.x & 63)) - 1ull))] = kk[u];
          }
        }
      }
      __syncthreads();
      const int lane = threadIdx.x & 63, c = bp.c, r = k - above - bp.above;
      const uint32_t v = lane < c ? small[lane] : 0u;
      int gt = 0, ge = 0;
      for (int j = 0; j < c; ++j) {
        const uint32_t w = (uint32_t)__builtin_amdgcn_readlane((int)v, j);
        gt += w > v;
        ge += w >= v;
      }
      const uint64_t hit = __ballot(lane < c && gt < r && r <= ge);
      const int l = __builtin_ctzll(hit);
      const int a = above + bp.above;
      return Kth{(uint32_t)__builtin_amdgcn_readlane((int)v, l),
                 a + __builtin_amdgcn_readlane(gt, l), a + __builtin_amdgcn_readlane(ge, l)};
    }
    above += bp.above;
  }
}

// A threshold key tau such that the count of keys >= tau is at least m when possible and
// at most `hard`, preferably at most `soft`; every key lies in [lo, hi].  Returns tau and
// that count.
__device__ __forceinline__ void local_threshold(const uint32_t* keys, int n, int m, int soft,
                                                int hard, uint32_t lo, uint32_t hi, const Lds& L,
                                                uint32_t& tau, int& count) {
  const int sh = range_shift(hi - lo);
  const BinPick bp = rank_bin(keys, n, lo, hi - lo, sh, m, L);
  const int tot = bp.above + bp.c;
  if (tot <= soft) {
    tau = lo + ((uint32_t)bp.d << sh);
    count = tot;
    return;
  }
  // the bin at the cut is crowded: cut at the exact m-th key instead
  __syncthreads();
  const Kth kt = radix_kth(keys, n, m, lo, hi, L);
  if (kt.ge <= hard) {
    tau = kt.T;
    count = kt.ge;
  } else {
    tau = kt.T + 1u;   // too many keys equal the m-th: keep only those above it
    count = kt.gt;
  }
}

// Stable selection of keys[0, n) in index order, one contiguous run per wave with ballot
// compaction: key i is taken if key > T, or key == T and fewer than `need` earlier keys equal
// to T were taken.  out(slot, i, key) for each taken key.  Each pass reads four 64-key
// chunks at once.
template <class Out>
__device__ __forceinline__ void emit_sel(const uint32_t* keys, int n, uint32_t T, int need,
                                         Out out, const Lds& L) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int chunk = ((n + NWAVE * 64 - 1) / (NWAVE * 64)) * 64;
  const int lo = min(n, wave * chunk), hi = min(n, lo + chunk);
  int gt = 0, eq = 0;
  for (int i0 = lo; i0 < hi; i0 += 256) {
    uint32_t k[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) k[u] = keys[min(i0 + 64 * u + lane, n - 1)];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool in = i0 + 64 * u + lane < hi;
      gt += __popcll(__ballot(in && k[u] > T));
      eq += __popcll(__ballot(in && k[u] == T));
    }
  }
  if (lane == 0) {
    L.wcnt[wave] = gt;
    L.wcnt[NWAVE + wave] = eq;
  }
  __syncthreads();
  int eq_base = 0, slot = 0;
  for (int w = 0; w < wave; ++w) {
    const int e = L.wcnt[NWAVE + w];
    slot += L.wcnt[w] + max(0, min(e, need - eq_base));
    eq_base += e;
  }
  __syncthreads();
  for (int i0 = lo; i0 < hi; i0 += 256) {
    uint32_t k[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) k[u] = keys[min(i0 + 64 * u + lane, n - 1)];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + 64 * u + lane;
      const bool in = i < hi;
      const bool is_eq = in && k[u] == T;
      const uint64_t eqb = __ballot(is_eq);
      const int eq_rank = eq_base + __popcll(eqb & ((1ull << lane) - 1ull));
      const bool take = (in && k[u] > T) || (is_eq && eq_rank < need);
      const uint64_t tb = __ballot(take);
      if (take) out(slot + __popcll(tb & ((1ull << lane) - 1ull)), i, k[u]);
      slot += __popcll(tb);
      eq_base += __popcll(eqb);
    }
  }
}

// ---------------------------------------------------------------------------------------
// Selection over keys held in registers: thread i holds the contiguous block of keys
// [E*i, E*i + E) of an LDS array (missing keys read as 0, below every real key), so every
// pass after the one LDS read works from registers, and a stable selection in index order
// needs only two workgroup scans.
// ---------------------------------------------------------------------------------------
// Exclusive scan of one int per thread over the workgroup (DPP within each wave); buf
// alternates between two halves of L.scan so that back-to-back scans need one barrier each.
__device__ __forceinline__ int wg_scan(int v, int buf, const Lds& L, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_scan_add(v);
  int* sc = L.scan + buf * NWAVE;
  if (lane == 63) sc[wave] = incl;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < NWAVE; ++w) {
    const int c = sc[w];
    before += w < wave ? c : 0;
    total += c;
  }
  return before + incl - v;
}

template <int E>
struct KeyBlock {
  static_assert(E % 4 == 0, "whole 16-byte reads");
  uint32_t k[E];
  int base, cnt;
  // keys[] must be 16-byte aligned and readable up to index E * NT.
  __device__ __forceinline__ void load(const uint32_t* keys, int n) {
    base = threadIdx.x * E;
    cnt = max(0, min(E, n - base));
#pragma unroll
    for (int e = 0; e < E; e += 4) {
      const u32x4 v = *(const u32x4*)(keys + base + e);
      k[e] = v.x;
      k[e + 1] = v.y;
      k[e + 2] = v.z;
      k[e + 3] = v.w;
    }
#pragma unroll
    for (int e = 0; e < E; ++e) k[e] = e < cnt ? k[e] : 0u;
  }
};

// Smallest and largest key of the block set (at least one key).
template <int E>
__device__ __forceinline__ void block_range(const KeyBlock<E>& b, const Lds& L, uint32_t& lo,
                                            uint32_t& hi) {
  uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    mn = min(mn, e < b.cnt ? b.k[e] : 0xffffffffu);
    mx = max(mx, b.k[e]);
  }
  mn = wave_min(mn);
  mx = wave_max(mx);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    L.range[wave] = mn;
    L.range[NWAVE + wave] = mx;
  }
  __syncthreads();
  lo = 0xffffffffu;
  hi = 0u;
#pragma unroll
  for (int w = 0; w < NWAVE; ++w) {
    lo = min(lo, L.range[w]);
    hi = max(hi, L.range[NWAVE + w]);
  }
}

// rank_bin over the block's keys; base must be above 0 (missing keys are 0).
template <int E>
__device__ __forceinline__ BinPick block_rank_bin(const KeyBlock<E>& b, uint32_t base,
                                                  uint32_t width, int sh, int r, const Lds& L) {
  int* hist = L.hist;
  __syncthreads();   // earlier readers of the histogram are done
  for (int i = threadIdx.x; i < kBins; i += NT) hist[i] = 0;
  __syncthreads();
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint32_t o = b.k[e] - base;
    if (o <= width) atomicAdd(&hist[o >> sh], 1);
  }
  __syncthreads();
  return find_in_hist(r, L);
}

// The k-th largest key of the block set when it lies in the bin [base, base + width] (base
// >= 1) that holds c <= 64 keys with `above` keys above it: the bin's keys are gathered into
// L.small and ranked within one wave.
template <int E>
__device__ __forceinline__ Kth block_bin_kth(const KeyBlock<E>& b, uint32_t base, uint32_t width,
                                             int above, int c, int k, const Lds& L) {
  const int lane = threadIdx.x & 63;
  if (threadIdx.x == 0) L.bcast[3] = 0;
  __syncthreads();
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool in = b.k[e] - base <= width;
    const uint64_t bl = __ballot(in);
    if (bl) {
      int at = 0;
      if (lane == 0) at = atomicAdd(&L.bcast[3], __popcll(bl));
      at = __builtin_amdgcn_readfirstlane(at);
      if (in) L.small[at + __popcll(bl & ((1ull << lane) - 1ull))] = b.k[e];
    }
  }
  __syncthreads();
  const int r = k - above;
  const uint32_t v = lane < c ? L.small[lane] : 0u;
  int gt = 0, ge = 0;
  for (int j = 0; j < c; ++j) {
    const uint32_t w = (uint32_t)__builtin_amdgcn_readlane((int)v, j);
    gt += w > v;
    ge += w >= v;
  }
  const uint64_t hit = __ballot(lane < c && gt < r && r <= ge);
  const int l = __builtin_ctzll(hit);
  return Kth{(uint32_t)__builtin_amdgcn_readlane((int)v, l), above + __builtin_amdgcn_readlane(gt, l),
             above + __builtin_amdgcn_readlane(ge, l)};
}

// The k-th largest key of the block set, with the counts above and at-or-above it.
template <int E>
__device__ __forceinline__ Kth block_kth(const KeyBlock<E>& b, int k, uint32_t lo, uint32_t hi,
                                         const Lds& L) {
  uint32_t base = lo, width = hi - lo;
  int above = 0;
  for (;;) {
    const int sh = range_shift(width);
    const BinPick bp = block_rank_bin(b, base, width, sh, k - above, L);
    base += (uint32_t)bp.d << sh;
    if (sh == 0) return Kth{base, above + bp.above, above + bp.above + bp.c};
    width = (1u << sh) - 1u;
    if (bp.c <= 64) return block_bin_kth(b, base, width, above + bp.above, bp.c, k, L);
    above += bp.above;
  }
}

// Stable selection in index order: key i is taken if key > T, or key == T and fewer than
// `need` earlier keys equal to T were taken.  out(slot, i, key) for each taken key.
template <int E, class Out>
__device__ __forceinline__ void block_emit(const KeyBlock<E>& b, uint32_t T, int need, Out out,
                                           const Lds& L) {
  int eq = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) eq += b.k[e] == T;
  int total;
  const int eq_base = wg_scan(eq, 0, L, total);
  int sel = 0, r = eq_base;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (b.k[e] > T) ++sel;
    else if (b.k[e] == T) { sel += r < need; ++r; }
  }
  int slot = wg_scan(sel, 1, L, total);
  r = eq_base;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    bool take = b.k[e] > T;
    if (b.k[e] == T) { take = r < need; ++r; }
    if (take) out(slot++, b.base + e, b.k[e]);
  }
}

__device__ __forceinline__ void pad_output(const IndexerParams& p, int t, int from) {
  for (int s = from + (int)threadIdx.x; s < p.K; s += NT) {
    p.out_idx[(size_t)t * p.K + s] = -1;
    if (p.out_score) p.out_score[(size_t)t * p.K + s] = 0.f;
  }
}

// ---------------------------------------------------------------------------------------
// Merge of a query's split candidates (run by the last split to arrive).
//
// Split r writes its candidates (key, position), in position order, to its own run of slots
// [r*rs, r*rs + count) of the query's candidate area (rs = cap rounded up to 4), zeroes the
// keys of the rest of the run's last 4-entry chunk, and writes its count to its header.  The
// merge reads the runs in split order as one list, the "virtual" list, in which every run
// takes whole chunks: entry v lies in the run r with pre[r] <= v < pre[r+1], where pre[r]
// sums the counts of the splits before r, each rounded up to 4.  Key 0 lies below every real
// key and marks the padding.  Split r covers positions [r*split, (r+1)*split), so the virtual
// list is in position order.  The merge finds the bin of the K_eff-th key by range-fitted radix passes over the
// list, gathers every entry at or above that bin in virtual order, finds the exact K_eff-th
// key T (and, among keys equal to T, the lower positions) within the gathered set, and
// writes the taken entries in gathered order: the output comes out sorted by position with
// no sort and no per-split bookkeeping.
// ---------------------------------------------------------------------------------------
struct MergeHdr {
  int n;              // length of the virtual list (a multiple of 4)
  int n_real;         // candidates of all runs
  uint32_t max_tau;   // largest split threshold
  uint32_t lo, hi;    // every candidate key lies in [lo, hi]
};

__device__ __forceinline__ uint32_t add_agent(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Split header words: emitted count, threshold, (unused), smallest and largest emitted key.
constexpr int kHdrWords = 8;

// Reduces the split headers of query t and writes the run starts pre[0 .. nsplit] to LDS
// (pre[nsplit] = the list's length).  Thread i reads the headers of a contiguous block of
// splits, so one workgroup scan yields the starts.
__device__ __forceinline__ MergeHdr load_headers(const IndexerParams& p, int t, int nsplit,
                                                 uint32_t* pre, const Lds& L) {
  constexpr int PER = kNSplitMax / NT;
  const uint32_t* hdr = p.hdr + (size_t)t * p.nsplit_max * kHdrWords;
  const int per = (nsplit + NT - 1) / NT;
  const int j0 = min(nsplit, per * (int)threadIdx.x), j1 = min(nsplit, j0 + per);
  uint32_t cnt[PER], tj[PER], lj[PER], hj[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const uint32_t* h = hdr + kHdrWords * (j0 + u);
    const bool in = j0 + u < j1;
    cnt[u] = in ? ld_agent(h) : 0u;
    tj[u] = in ? ld_agent(h + 1) : 0u;
    lj[u] = in ? ld_agent(h + 3) : 0xffffffffu;
    hj[u] = in ? ld_agent(h + 4) : 0u;
  }
  int c = 0, c4 = 0;
  uint32_t tau = 0u, lo = 0xffffffffu, hi = 0u;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    c += (int)cnt[u];
    c4 += (int)((cnt[u] + 3u) & ~3u);
    tau = max(tau, tj[u]);
    if (cnt[u]) {
      lo = min(lo, lj[u]);
      hi = max(hi, hj[u]);
    }
  }
  int total;
  int b = wg_scan(c4, 0, L, total);
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    if (j0 + u < j1) pre[j0 + u] = (uint32_t)b;
    b += (int)((cnt[u] + 3u) & ~3u);
  }
  if (threadIdx.x == 0) pre[nsplit] = (uint32_t)total;
  c = wave_scan_add(c);
  c = __builtin_amdgcn_readlane(c, 63);
  tau = wave_max(tau);
  lo = wave_min(lo);
  hi = wave_max(hi);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    L.wcnt[wave] = (int)tau;
    L.wcnt[NWAVE + wave] = c;
    L.range[wave] = lo;
    L.range[NWAVE + wave] = hi;
  }
  __syncthreads();
  MergeHdr h;
  h.n = total;
  h.n_real = 0;
  h.max_tau = 0u;
  h.lo = 0xffffffffu;
  h.hi = 0u;
#pragma unroll
  for (int w = 0; w < NWAVE; ++w) {
    h.max_tau = max(h.max_tau, (uint32_t)L.wcnt[w]);
    h.n_real += L.wcnt[NWAVE + w];
    h.lo = min(h.lo, L.range[w]);
    h.hi = max(h.hi, L.range[NWAVE + w]);
  }
  return h;
}

// Runs holding the virtual indices v[u] (v[u] < pre[nsplit]; entries with v[u] < 0 are left
// at run 0): the largest r with pre[r] <= v, and pre[r], by a branch-free binary search whose
// LDS reads for all U indices are in flight together.
template <int U>
__device__ __forceinline__ void runs_of(const uint32_t* pre, int nsplit, const int (&v)[U],
                                        int (&r)[U], int (&pr)[U]) {
  int step = 1;
  while (2 * step < nsplit) step *= 2;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    r[u] = 0;
    pr[u] = 0;
  }
  for (; step >= 1; step >>= 1) {
    uint32_t x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = r[u] + step < nsplit ? pre[r[u] + step] : 0xffffffffu;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool up = v[u] >= 0 && x[u] <= (uint32_t)v[u];
      r[u] += up ? step : 0;
      pr[u] = up ? (int)x[u] : pr[u];
    }
  }
}

// Slot of virtual index v in the query's candidate area (run stride rs).
__device__ __forceinline__ int run_slot(const uint32_t* pre, int nsplit, int rs, int v) {
  int vv[1] = {v}, r[1], pr[1];
  runs_of<1>(pre, nsplit, vv, r, pr);
  return r[0] * rs + v - pr[0];
}

// Copies the virtual list (n entries, a multiple of 4) into LDS: keys to lk and, when lp is not
// null, positions to lp, with agent-scope direct-to-LDS loads of 16 bytes per lane.  Every run
// takes whole 4-entry chunks.  Long runs (48 entries or more on average) are copied one run
// per load (lane l: chunk l of the run; wave w copies runs w, w + 4, ...).  Short runs would
// leave most lanes of such a load idle, so then a load fills 64 consecutive chunks of the list
// instead, each lane finding its chunk's run by binary search.
__device__ __forceinline__ void stage_runs(const uint32_t* gk, const int32_t* gp, int rs,
                                           int nsplit, int n, const uint32_t* pre, uint32_t* lk,
                                           int32_t* lp) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int per = lp ? 2 : 1;
  int issued = 0;
  auto throttle = [&]() {
    issued += per;
    if (issued >= 56) {   // at most 56 loads in flight: inside the 6-bit load counter
      wait_vmcnt<40>();
      issued = 40;
    }
  };
  if (n >= 48 * nsplit) {
    for (int r0 = wave; r0 < nsplit; r0 += 64 * NWAVE) {
      // lane l: the bounds of run r0 + 4 l
      const int rl = min(r0 + NWAVE * lane, nsplit - 1);
      const int bl = (int)pre[rl];
      const int el = (int)pre[rl + 1];
      const int nr = min(64, (nsplit - r0 + NWAVE - 1) / NWAVE);
      for (int u = 0; u < nr; ++u) {
        const int r = r0 + NWAVE * u;
        const int b = __builtin_amdgcn_readlane(bl, u);
        const int c = __builtin_amdgcn_readlane(el, u) - b;
        for (int i = 0; i < c; i += 256) {
          if (4 * lane < c - i) {
            const uint32_t src = 4u * (uint32_t)(r * rs + i + 4 * lane);
            load_to_lds<16, true>(gk, src, lds_addr(lk + b + i));
            if (lp) load_to_lds<16, true>(gp, src, lds_addr(lp + b + i));
          }
          throttle();
        }
      }
    }
  } else {
    constexpr int B = 4;
    const int nc = n >> 2;
    for (int i0 = 0; 64 * (wave + NWAVE * i0) < nc; i0 += B) {
      int v[B], r[B], pr[B];
#pragma unroll
      for (int u = 0; u < B; ++u) {
        const int c = 64 * (wave + NWAVE * (i0 + u)) + lane;
        v[u] = c < nc ? 4 * c : -1;
      }
      runs_of<B>(pre, nsplit, v, r, pr);
#pragma unroll
      for (int u = 0; u < B; ++u) {
        const int cb = 64 * (wave + NWAVE * (i0 + u));
        if (cb >= nc) break;
        if (v[u] >= 0) {
          const uint32_t src = 4u * (uint32_t)(r[u] * rs + v[u] - pr[u]);
          load_to_lds<16, true>(gk, src, lds_addr(lk + 4 * cb));
          if (lp) load_to_lds<16, true>(gp, src, lds_addr(lp + 4 * cb));
        }
        throttle();
      }
    }
  }
  wait_vmcnt<0>();
}

// Row-major selection over entries [0, n) whose keys come from key_of(i) (0: no entry).
// Passes read four rows per thread at once so that global reads overlap.
template <class KeyOf>
__device__ __forceinline__ BinPick rm_rank_bin(int n, KeyOf key_of, uint32_t base,
                                               uint32_t width, int sh, int r, const Lds& L) {
  int* hist = L.hist;
  __syncthreads();   // earlier readers of the histogram are done
  for (int i = threadIdx.x; i < kBins; i += NT) hist[i] = 0;
  __syncthreads();
  for (int i0 = threadIdx.x; i0 < n; i0 += 4 * NT) {
    uint32_t k[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) k[u] = i0 + u * NT < n ? key_of(i0 + u * NT) : 0u;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t o = k[u] - base;
      if ((k[u] != 0u) & (o <= width)) atomicAdd(&hist[o >> sh], 1);
    }
  }
  __syncthreads();
  return find_in_hist(r, L);
}

// Among the c <= 64 keys of the entries that lie in [base, base + width] (base >= 1): the
// r-th largest, with the counts above it and at or above it among them.  Each wave compacts
// the keys of its rows into its own 64-entry list (L.psum); every wave then ranks their
// concatenation.
template <class KeyOf>
__device__ __forceinline__ Kth rank_few(int n, KeyOf key_of, uint32_t base, uint32_t width,
                                        int c, int r, const Lds& L) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t* mine = (uint32_t*)L.psum + 64 * wave;
  int cnt = 0;
  __syncthreads();   // every wave is done with L.psum and L.wcnt
  for (int i0 = 64 * wave; i0 < n; i0 += 4 * NT) {
    uint32_t kk[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * NT + lane;
      kk[u] = i < n ? key_of(i) : 0u;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool in = (kk[u] != 0u) & (kk[u] - base <= width);
      const uint64_t bl = __ballot(in);
      if (in) mine[cnt + __popcll(bl & ((1ull << lane) - 1ull))] = kk[u];
      cnt += __popcll(bl);
    }
  }
  if (lane == 0) L.wcnt[wave] = cnt;
  __syncthreads();
  int lw = lane, w = 0;
#pragma unroll
  for (int q = 0; q < NWAVE - 1; ++q)
    if (w == q && lw >= L.wcnt[q]) { lw -= L.wcnt[q]; w = q + 1; }
  const uint32_t v = lane < c ? ((const uint32_t*)L.psum)[64 * w + lw] : 0u;
  int gt = 0, ge = 0;
  for (int j = 0; j < c; ++j) {
    const uint32_t x = (uint32_t)__builtin_amdgcn_readlane((int)v, j);
    gt += x > v;
    ge += x >= v;
  }
  const uint64_t hit = __ballot(lane < c && gt < r && r <= ge);
  const int l = __builtin_ctzll(hit);
  return Kth{(uint32_t)__builtin_amdgcn_readlane((int)v, l), __builtin_amdgcn_readlane(gt, l),
             __builtin_amdgcn_readlane(ge, l)};
}

// Range-fitted radix passes over the entries, narrowing to the bin that holds the k-th
// largest key until that bin is a single key value or holds at most 64 keys.  Returns the
// bin [base, base + width], the count above it and the count in it.
struct Narrowed { uint32_t base, width; int above, c; };
template <class KeyOf>
__device__ __forceinline__ Narrowed rm_narrow(int n, KeyOf key_of, int k, uint32_t lo,
                                              uint32_t hi, const Lds& L) {
  Narrowed nw{lo, hi - lo, 0, 0};
  for (;;) {
    const int sh = range_shift(nw.width);
    const BinPick bp = rm_rank_bin(n, key_of, nw.base, nw.width, sh, k - nw.above, L);
    nw.base += (uint32_t)bp.d << sh;
    nw.width = sh ? (1u << sh) - 1u : 0u;
    nw.above += bp.above;
    nw.c = bp.c;
    if (sh == 0 || bp.c <= 64) return nw;
  }
}

// The k-th largest key among the entries, as radix_kth (every key in [lo, hi], lo >= 1).
template <class KeyOf>
__device__ __forceinline__ Kth rm_kth(int n, KeyOf key_of, int k, uint32_t lo, uint32_t hi,
                                      const Lds& L) {
  const Narrowed nw = rm_narrow(n, key_of, k, lo, hi, L);
  if (nw.width == 0) return Kth{nw.base, nw.above, nw.above + nw.c};
  const Kth kt = rank_few(n, key_of, nw.base, nw.width, nw.c, k - nw.above, L);
  return Kth{kt.T, nw.above + kt.gt, nw.above + kt.ge};
}

// Compacts the entries with pred(key, v) into the selection area, keeping their virtual
// order: thread i scans the contiguous block [E*i, E*i + E) of the list (E odd, so that the
// LDS reads of a wave fall in distinct banks), counts, takes its offset from a workgroup
// scan, then writes keys and virtual indices; pos_batch(v, ps) then turns U virtual indices
// per thread into positions with all reads in flight.  Returns the count (at most kSelCap
// are stored).
constexpr int kGatherU = (kSelCap + NT - 1) / NT;
template <class KeyOf, class Pred, class PosBatch>
__device__ __forceinline__ int gather_ordered(int n, KeyOf key_of, Pred pred, PosBatch pos_batch,
                                              const Lds& L) {
  const int E = ((n + NT - 1) / NT) | 1;
  const int b0 = min(n, E * (int)threadIdx.x), b1 = min(n, b0 + E);
  int c = 0;
  for (int i0 = b0; i0 < b1; i0 += 4) {
    uint32_t k[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) k[u] = i0 + u < b1 ? key_of(i0 + u) : 0u;
#pragma unroll
    for (int u = 0; u < 4; ++u) c += (int)((k[u] != 0u) & pred(k[u], i0 + u));
  }
  int total;
  __syncthreads();   // earlier readers of L.scan are done
  int at = wg_scan(c, 0, L, total);
  for (int i0 = b0; i0 < b1; i0 += 4) {
    uint32_t k[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) k[u] = i0 + u < b1 ? key_of(i0 + u) : 0u;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if ((k[u] != 0u) & pred(k[u], i0 + u)) {
        if (at < kSelCap) {
          L.sel_key[at] = k[u];
          L.sel_pos[at] = i0 + u;
        }
        ++at;
      }
    }
  }
  __syncthreads();
  const int ns = min(total, kSelCap);
  int v[kGatherU];
  int32_t ps[kGatherU];
#pragma unroll
  for (int u = 0; u < kGatherU; ++u) {
    const int q = threadIdx.x + u * NT;
    v[u] = q < ns ? L.sel_pos[q] : -1;
  }
  pos_batch(v, ps);
#pragma unroll
  for (int u = 0; u < kGatherU; ++u) {
    const int q = threadIdx.x + u * NT;
    if (q < ns) L.sel_pos[q] = ps[u];
  }
  __syncthreads();
  return total;
}

// Selection and output over the virtual list, keys from key_of(v), positions from pos_of(v)
// one at a time or pos_batch for a batch.  Returns false (writing nothing) when a split's
// threshold lies above the K_eff-th key T.
template <class KeyOf, class PosOf, class PosBatch>
__device__ __forceinline__ bool merge_select(const IndexerParams& p, int t, int K_eff,
                                             const MergeHdr& mh, KeyOf key_of, PosOf pos_of,
                                             PosBatch pos_batch, const Lds& L, uint32_t& T,
                                             int& gt, bool& enough) {
  const int n = mh.n;
  enough = mh.n_real >= K_eff;
  T = 0u;
  gt = 0;
  int ge = 0;
  uint32_t pmax = 0xffffffffu;
  int ns;   // entries in the selection area, in virtual order: the selection and maybe a few more
  auto sel_key = [&](int q) { return L.sel_key[q]; };
  if (!enough) {
    if (mh.max_tau != 0u) return false;
    ns = gather_ordered(n, key_of, [](uint32_t, int) { return true; }, pos_batch, L);
  } else {
    // one radix pass usually isolates a bin of a few keys holding the K_eff-th; every key at
    // or above that bin is gathered, and the exact K_eff-th is found among them
    const Narrowed nw = rm_narrow(n, key_of, K_eff, mh.lo, mh.hi, L);
    if (nw.above + nw.c <= kSelCap) {
      ns = gather_ordered(n, key_of, [&](uint32_t k, int) { return k >= nw.base; }, pos_batch, L);
      if (nw.width == 0) {
        T = nw.base;
        gt = nw.above;
        ge = nw.above + nw.c;
      } else {
        const Kth kt = rank_few(ns, sel_key, nw.base, nw.width, nw.c, K_eff - nw.above, L);
        T = kt.T;
        gt = nw.above + kt.gt;
        ge = nw.above + kt.ge;
      }
      if (mh.max_tau > T) return false;
      const int need = K_eff - gt;
      if (ge - gt > need) {
        // among keys equal to T the lower positions win: the need-th smallest tied position
        auto tied = [&](int q) -> uint32_t {
          return L.sel_key[q] == T ? ~(uint32_t)L.sel_pos[q] : 0u;
        };
        pmax = ~rm_kth(ns, tied, need, 0x80000000u, 0xffffffffu, L).T;
      }
    } else {
      // a crowd of equal keys: the exact selection over the whole list, then its entries
      const Kth kt = rm_kth(n, key_of, K_eff, mh.lo, mh.hi, L);
      T = kt.T;
      gt = kt.gt;
      ge = kt.ge;
      if (mh.max_tau > T) return false;
      const int need = K_eff - gt;
      if (ge - gt > need) {
        auto tied = [&](int i) -> uint32_t { return key_of(i) == T ? ~(uint32_t)pos_of(i) : 0u; };
        pmax = ~rm_kth(n, tied, need, 0x80000000u, 0xffffffffu, L).T;
      }
      const uint32_t TT = T, PM = pmax;
      ns = gather_ordered(n, key_of,
                          [&](uint32_t k, int i) { return k > TT || (k == TT && (uint32_t)pos_of(i) <= PM); },
                          pos_batch, L);
    }
  }
  ns = min(ns, kSelCap);
  // Output.  The selection area holds, in position order, every taken entry and at most 64
  // more (keys of the K_eff-th key's bin below T, or equal to T past pmax): taken are the
  // keys above T and those equal to T at positions up to pmax (T = 0: every entry).  Thread
  // i takes a contiguous block of the area; a workgroup scan of the taken counts gives the
  // output slots.
  constexpr int EMAX = kGatherU | 1;
  const int E = ((ns + NT - 1) / NT) | 1;
  const int b0 = min(ns, E * (int)threadIdx.x), b1 = min(ns, b0 + E);
  uint32_t k[EMAX];
  int32_t ps[EMAX];
  bool tk[EMAX];
  int c = 0;
#pragma unroll
  for (int u = 0; u < EMAX; ++u) {
    const int q = max(0, min(b0 + u, ns - 1));
    k[u] = L.sel_key[q];
    ps[u] = L.sel_pos[q];
  }
#pragma unroll
  for (int u = 0; u < EMAX; ++u) {
    tk[u] = (b0 + u < b1) & ((k[u] > T) | ((k[u] == T) & ((uint32_t)ps[u] <= pmax)));
    c += tk[u];
  }
  int total;
  __syncthreads();   // earlier readers of L.scan are done
  int slot = wg_scan(c, 1, L, total);
#pragma unroll
  for (int u = 0; u < EMAX; ++u) {
    if (tk[u]) {
      if (slot < K_eff) {
        p.out_idx[(size_t)t * p.K + slot] = ps[u];
        if (p.out_score) p.out_score[(size_t)t * p.K + slot] = key_to_float(k[u]);
      }
      ++slot;
    }
  }
  pad_output(p, t, min(total, K_eff));
  if (threadIdx.x == 0) st_agent(p.counters + t, 0u);
  return true;
}

// ---------------------------------------------------------------------------------------
// Selection over a list in LDS read four entries per lane (one 16-byte read), for the merge:
// keys[0, n) with n a multiple of 4 and keys 16-byte aligned; key 0 marks padding and lies
// below every real key.  Each pass issues one LDS read per four entries, so the merge's
// passes cost a quarter of the instructions of one-entry-per-lane loops.
// ---------------------------------------------------------------------------------------
// rank_bin over the list (base >= 1, so padding never counts).
__device__ __forceinline__ BinPick lst_rank_bin(const uint32_t* keys, int n, uint32_t base,
                                                uint32_t width, int sh, int r, const Lds& L) {
  int* hist = L.hist;
  __syncthreads();   // earlier readers of the histogram are done
  for (int i = threadIdx.x; i < kBins / 4; i += NT) *(int4*)(hist + 4 * i) = int4{0, 0, 0, 0};
  __syncthreads();
  const int nc = n >> 2;
#pragma unroll 2
  for (int c = threadIdx.x; c < nc; c += NT) {
    const u32x4 k = *(const u32x4*)(keys + 4 * c);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t o = k[u] - base;
      if (o <= width) atomicAdd(&hist[o >> sh], 1);
    }
  }
  __syncthreads();
  return find_in_hist(r, L);
}

// The k-th largest key of the list, as radix_kth (every real key in [lo, hi], lo >= 1).
__device__ __forceinline__ Kth lst_kth(const uint32_t* keys, int n, int k, uint32_t lo,
                                       uint32_t hi, const Lds& L) {
  uint32_t base = lo, width = hi - lo;
  int above = 0;
  const int lane = threadIdx.x & 63, nc = n >> 2;
  for (;;) {
    const int sh = range_shift(width);
    const BinPick bp = lst_rank_bin(keys, n, base, width, sh, k - above, L);
    base += (uint32_t)bp.d << sh;
    if (sh == 0) return Kth{base, above + bp.above, above + bp.above + bp.c};
    width = (1u << sh) - 1u;
    if (bp.c > 64) {
      above += bp.above;
      continue;
    }
    // the c <= 64 keys of the bin, gathered into L.small and ranked within one wave
    if (threadIdx.x == 0) L.bcast[3] = 0;
    __syncthreads();
    for (int c = threadIdx.x; c < nc; c += NT) {
      const u32x4 kk = *(const u32x4*)(keys + 4 * c);
      int m = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) m += kk[u] - base <= width;
      if (m) {
        int at = atomicAdd(&L.bcast[3], m);
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (kk[u] - base <= width) L.small[at++] = kk[u];
      }
    }
    __syncthreads();
    const int c = bp.c, r = k - above - bp.above;
    const uint32_t v = lane < c ? L.small[lane] : 0u;
    int gt = 0, ge = 0;
    for (int j = 0; j < c; ++j) {
      const uint32_t w = (uint32_t)__builtin_amdgcn_readlane((int)v, j);
      gt += w > v;
      ge += w >= v;
    }
    const uint64_t hit = __ballot(lane < c && gt < r && r <= ge);
    const int l = __builtin_ctzll(hit);
    const int a = above + bp.above;
    return Kth{(uint32_t)__builtin_amdgcn_readlane((int)v, l),
               a + __builtin_amdgcn_readlane(gt, l), a + __builtin_amdgcn_readlane(ge, l)};
  }
}

// Stable selection of the list in index order: entry i is taken if its key is above T, or
// equal to T and fewer than `need` earlier entries equal to T were taken; taken entry number
// s (in index order) writes pos[i] to out[s] (s < limit).  Wave w owns a contiguous range of
// 4-entry chunks; within one step of 64 chunks a packed exclusive scan of the per-lane
// (taken above T, equal to T) counts gives every lane its slots.
__device__ __forceinline__ void lst_emit_range(const uint32_t* keys, const int32_t* pos, int c0,
                                               int c1, uint32_t T, int need, int32_t* out,
                                               float* out_score, int limit, int slot, int eq);
__device__ __forceinline__ void lst_emit(const uint32_t* keys, const int32_t* pos, int n,
                                         uint32_t T, int need, int32_t* out, float* out_score,
                                         int limit, const Lds& L) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nc = n >> 2;
  const int cpw = (nc + NWAVE - 1) / NWAVE;
  const int c0 = min(nc, wave * cpw), c1 = min(nc, c0 + cpw);
  int g = 0, e = 0;
  for (int c = c0 + lane; c < c1; c += 64) {
    const u32x4 k = *(const u32x4*)(keys + 4 * c);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      g += k[u] > T;
      e += k[u] == T;
    }
  }
  g = wave_scan_add(g);
  e = wave_scan_add(e);
  if (lane == 63) {
    L.wcnt[wave] = g;
    L.wcnt[NWAVE + wave] = e;
  }
  __syncthreads();
  int slot = 0, eq = 0;   // taken entries and ties before this wave's range
  for (int w = 0; w < wave; ++w) {
    const int ew = L.wcnt[NWAVE + w];
    slot += L.wcnt[w] + max(0, min(ew, need - eq));
    eq += ew;
  }
  __syncthreads();
  lst_emit_range(keys, pos, c0, c1, T, need, out, out_score, limit, slot, eq);
}

// The emission of lst_emit over this wave's chunks [c0, c1), given the entries taken (slot)
// and the keys equal to T (eq) before them.
__device__ __forceinline__ void lst_emit_range(const uint32_t* keys, const int32_t* pos, int c0,
                                               int c1, uint32_t T, int need, int32_t* out,
                                               float* out_score, int limit, int slot, int eq) {
  const int lane = threadIdx.x & 63;
  for (int cb = c0; cb < c1; cb += 64) {
    const int c = cb + lane;
    u32x4 k = {0u, 0u, 0u, 0u};
    if (c < c1) k = *(const u32x4*)(keys + 4 * c);
    int gl = 0, el = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      gl += k[u] > T;
      el += k[u] == T;
    }
    // exclusive prefix of (above T, equal to T) over the lanes, packed 16:16 (<= 256 each)
    const int incl = wave_scan_add(gl | (el << 16));
    const int excl = incl - (gl | (el << 16));
    const int tot = __builtin_amdgcn_readlane(incl, 63);
    int gb = excl & 0xffff, eb = eq + (excl >> 16);
    int s = slot + gb + max(0, min(eb - eq, need - eq));
    if (gl | el) {
      const i32x4 ps = *(const i32x4*)(pos + 4 * c);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        bool take = k[u] > T;
        if (k[u] == T) take = eb++ < need;
        if (take) {
          if (s < limit) {
            out[s] = ps[u];
            if (out_score) out_score[s] = key_to_float(k[u]);
          }
          ++s;
        }
      }
    }
    slot += (tot & 0xffff) + max(0, min(tot >> 16, need - eq));
    eq += tot >> 16;
  }
}

// Selection over the staged list (keys fk, positions fp, in list order = position order),
// with the LDS-resident, ballot-based routines of the single-split path: radix_kth finds the
// exact K_eff-th key T with the counts above it (gt) and at or above it (ge); when every
// split's threshold is at or below T the candidates provably hold the answer, and emit_sel
// takes, in list order, every key above T and the first K_eff - gt keys equal to T, which
// are the lowest positions among the tied ones.  The emission order is the output order.
// Padding entries (key 0) lie below every real key and are never taken.  Returns 1 when the
// output is written, 0 when a split's threshold lies above T (the caller re-scores), -1 when
// the list does not qualify.
__device__ __forceinline__ int merge_fast(const IndexerParams& p, int t, int K_eff,
                                          const MergeHdr& mh, const uint32_t* fk,
                                          const int32_t* fp, const Lds& L, uint32_t& T, int& gt,
                                          bool& enough) {
  enough = mh.n_real >= K_eff;
  if (!enough) return -1;
  int32_t* out = p.out_idx + (size_t)t * p.K;
  float* out_s = p.out_score ? p.out_score + (size_t)t * p.K : nullptr;
  const int n = mh.n, nc = n >> 2;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // One radix pass finds the bin of the K_eff-th key.  When that bin holds at most 64 keys,
  // one more pass over the list both gathers them (with their wave) and counts, per wave, the
  // keys above the bin; the bin's keys ranked within a wave then give T and every wave's
  // counts above and at T, so the output's count pass is not needed.  Otherwise lst_kth
  // narrows the bin and lst_emit counts.
  if (threadIdx.x == 0) L.bcast[3] = 0;
  const uint32_t width = mh.hi - mh.lo;
  const int sh = range_shift(width);
  const BinPick bp = lst_rank_bin(fk, n, mh.lo, width, sh, K_eff, L);
  tl_stamp(p.tl, kTlIndexer, kTlKthBin);
  if (sh == 0 || bp.c > 64) {
    const Kth kt = lst_kth(fk, n, K_eff, mh.lo, mh.hi, L);
    T = kt.T;
    gt = kt.gt;
    tl_stamp(p.tl, kTlIndexer, kTlKth);
    if (mh.max_tau > T) return 0;
    lst_emit(fk, fp, n, T, K_eff - gt, out, out_s, K_eff, L);
  } else {
    const uint32_t blo = mh.lo + ((uint32_t)bp.d << sh), bw = (1u << sh) - 1u;
    uint32_t* const bin_wave = L.small_w;
    const int cpw = (nc + NWAVE - 1) / NWAVE;
    const int c0 = min(nc, wave * cpw), c1 = min(nc, c0 + cpw);
    int above = 0;
    for (int c = c0 + lane; c < c1; c += 64) {
      const u32x4 k = *(const u32x4*)(fk + 4 * c);
      int m = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        above += k[u] - blo > bw && k[u] > blo;   // above the bin (key 0 padding is below it)
        m += k[u] - blo <= bw;
      }
      if (m) {
        int at = atomicAdd(&L.bcast[3], m);
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (k[u] - blo <= bw) {
            L.small[at] = k[u];
            bin_wave[at++] = (uint32_t)wave;
          }
      }
    }
    above = __builtin_amdgcn_readlane(wave_scan_add(above), 63);
    if (lane == 0) L.wcnt[wave] = above;
    __syncthreads();
    const int cb = bp.c, r = K_eff - bp.above;
    const uint32_t v = lane < cb ? L.small[lane] : 0u;
    const int vw = lane < cb ? (int)bin_wave[lane] : -1;
    int g = 0, ge = 0;
    for (int j = 0; j < cb; ++j) {
      const uint32_t w = (uint32_t)__builtin_amdgcn_readlane((int)v, j);
      g += w > v;
      ge += w >= v;
    }
    const uint64_t hit = __ballot(lane < cb && g < r && r <= ge);
    const int l = __builtin_ctzll(hit);
    T = (uint32_t)__builtin_amdgcn_readlane((int)v, l);
    gt = bp.above + __builtin_amdgcn_readlane(g, l);
    tl_stamp(p.tl, kTlIndexer, kTlKth);
    if (mh.max_tau > T) return 0;
    const int need = K_eff - gt;
    int slot = 0, eq = 0;   // taken entries and ties before this wave's range
    for (int w = 0; w < wave; ++w) {
      const int gw = L.wcnt[w] + __popcll(__ballot(vw == w && v > T));
      const int ew = __popcll(__ballot(vw == w && v == T));
      slot += gw + max(0, min(ew, need - eq));
      eq += ew;
    }
    lst_emit_range(fk, fp, c0, c1, T, need, out, out_s, K_eff, slot, eq);
  }
  pad_output(p, t, K_eff);
  if (threadIdx.x == 0) st_agent(p.counters + t, 0u);
  tl_stamp(p.tl, kTlIndexer, kTlMerged);
  return 1;
}

// Run starts from the headers, then the virtual list staged in LDS when it fits (keys;
// positions too when there is room), then the selection.  T, gt and enough are kept for the
// re-scoring of failing splits.
template <int MODE>
__device__ __forceinline__ bool merge(const IndexerParams& p, int t, int K_eff, int nsplit,
                                      const Lds& L, uint32_t& T, int& gt, bool& enough) {
  constexpr int FW = flat_words<MODE>();
  constexpr int RW = region_bytes<MODE>() / 4;
  const int pw = (nsplit + 4) & ~3;   // pre[0 .. nsplit], whole 16-byte words
  uint32_t* pre = (uint32_t*)L.region + RW - pw;   // at the region's end
  const MergeHdr mh = load_headers(p, t, nsplit, pre, L);
  tl_stamp(p.tl, kTlIndexer, kTlHeaders);
  const int rs = p.rs;
  const size_t qb = (size_t)t * p.nsplit_max * rs;
  const uint32_t* gk = p.cand_key + qb;
  const int32_t* gp = p.cand_pos + qb;
  const int n = mh.n;
  // the list is staged in LDS when it fits (keys; positions too when there is room), else
  // read from the runs in global memory
  auto gkey = [&](int v) { return ld_agent(gk + run_slot(pre, nsplit, rs, v)); };
  auto gpos = [&](int v) { return ld_agent(gp + run_slot(pre, nsplit, rs, v)); };
  auto gpos_batch = [&](const int (&v)[kGatherU], int32_t (&ps)[kGatherU]) {
    int r[kGatherU], pr[kGatherU];
    runs_of<kGatherU>(pre, nsplit, v, r, pr);
#pragma unroll
    for (int u = 0; u < kGatherU; ++u)
      ps[u] = v[u] >= 0 ? ld_agent(gp + r[u] * rs + v[u] - pr[u]) : 0;
  };
  if (mh.n_real >= K_eff && 2 * n <= RW - pw) {
    // merge_fast needs no selection area: keys and positions from the region's start
    uint32_t* fk = (uint32_t*)L.region;
    int32_t* fp = (int32_t*)(fk + n);
    stage_runs(gk, gp, rs, nsplit, n, pre, fk, fp);
    __syncthreads();
    tl_stamp(p.tl, kTlIndexer, kTlStaged);
    return merge_fast(p, t, K_eff, mh, fk, fp, L, T, gt, enough) == 1;
  }
  // (here merge_fast would not apply: too few candidates, or a list too long for positions)
  if (n > FW - pw) return merge_select(p, t, K_eff, mh, gkey, gpos, gpos_batch, L, T, gt, enough);
  const bool pos_in = 2 * n <= FW - pw;
  uint32_t* fk = L.flat;
  int32_t* fp = (int32_t*)(fk + n);
  stage_runs(gk, gp, rs, nsplit, n, pre, fk, pos_in ? fp : nullptr);
  __syncthreads();
  auto lkey = [&](int v) { return fk[v]; };
  if (pos_in) {
    auto lpos = [&](int v) { return fp[v]; };
    auto lpos_batch = [&](const int (&v)[kGatherU], int32_t (&ps)[kGatherU]) {
#pragma unroll
      for (int u = 0; u < kGatherU; ++u) ps[u] = v[u] >= 0 ? fp[v[u]] : 0;
    };
    return merge_select(p, t, K_eff, mh, lkey, lpos, lpos_batch, L, T, gt, enough);
  }
  return merge_select(p, t, K_eff, mh, lkey, gpos, gpos_batch, L, T, gt, enough);
}

// ---------------------------------------------------------------------------------------
// Kernel.  The scorer has one call site: the loop first scores this workgroup's own split;
// only the merging workgroup of a query whose split thresholds failed to certify comes back
// to it, to re-score each failing split and take its exact local Top-K.
// ---------------------------------------------------------------------------------------
// One work item: split j of query t (scoring, candidate emission, and the merge when it is
// the query's last split to arrive).  With prescored the split's scores are already in
// L.keys, klo0 and khi0 their smallest and largest key.  phase 1 stops after the arrival and
// returns whether this workgroup must merge; phase 3 stops before it (the caller drains the
// stores and arrives); phase 2 does the merge (and the re-scoring it may need); phase 0 does
// everything.  Every return is uniform over the workgroup.
template <int MODE>
__device__ __forceinline__ bool run_item(const IndexerParams& p, int t, int j, const Lds& L,
                                         const Lds& Lm, bool prescored = false,
                                         uint32_t klo0 = 0u, uint32_t khi0 = 0u, int phase = 0) {
  const int split = p.split;
  const int cap = min(split, p.K);
  const int V = min(p.q_vis[t], p.max_visible);
  if (V <= 0) {
    if (j == 0) pad_output(p, t, 0);
    return false;
  }
  const int nsplit = (V + split - 1) / split;
  if (j >= nsplit) return false;
  const int seq = p.q_seq[t];
  const int K_eff = min(p.K, V);
  tl_put(p.tl, kTlIndexer, kTlItem, ((uint64_t)t << 16) | (uint32_t)j);

  const GenericSmem* gsp = nullptr;
  if constexpr (MODE == 0) {
    __shared__ GenericSmem gs;
    const int HD = p.H * p.D;
    for (int i = threadIdx.x; i < HD; i += NT)
      gs.q[i] = load_elem(p.q, p.q_dtype, (int64_t)t * HD + i);
    for (int i = threadIdx.x; i < p.H; i += NT) gs.w[i] = p.w[(size_t)t * p.H + i];
    if (p.k_dtype == kDtMX) {
      // MXFP8 keys: the query is quantized too, per head and group of 32 dims (one group per
      // thread), and replaced by its dequantized values (exact in fp32 down to 2^-149)
      __syncthreads();
      for (int g = threadIdx.x; g < HD / 32; g += NT) {
        float amax = 0.f;
        for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(gs.q[32 * g + i]));
        const uint32_t sb = mx_scale_byte(amax);
        for (int i = 0; i < 32; ++i)
          gs.q[32 * g + i] = (float)ldexp((double)fp8_e4m3_to_f32(f32_to_fp8_e4m3(gs.q[32 * g + i] * mx_inv_scale(sb))),
                                          (int)sb - 127);
      }
    }
    gsp = &gs;
  }
  __syncthreads();

  int cur = j;            // split to score
  bool refill = false;    // re-scoring failing splits for this query's merge
  uint32_t T = 0u;
  int gt = 0;
  bool enough = false;
  // The next split that fails the merge's threshold after split `from`, or -1.  The headers
  // are read again from the workspace: their LDS copy shares memory with the scorer's ring.
  auto next_failing = [&](int from) {
    int nxt = -1;
    for (int jj = from + 1; jj < nsplit && nxt < 0; ++jj) {
      const uint32_t tau = ld_agent(p.hdr + ((size_t)t * p.nsplit_max + jj) * kHdrWords + 1);
      if (enough ? (tau > T) : (tau != 0u)) nxt = jj;
    }
    nxt = __builtin_amdgcn_readfirstlane(nxt);   // same value in every lane
    wait_all_memory();
    __syncthreads();
    return nxt;
  };
  if (phase == 2) {
    if (merge<MODE>(p, t, K_eff, nsplit, Lm, T, gt, enough)) return false;
    refill = true;
    cur = next_failing(-1);
    if (cur < 0) {
      merge<MODE>(p, t, K_eff, nsplit, Lm, T, gt, enough);   // certified
      return false;
    }
  }
  for (;;) {
    const int start = cur * split, len = min(split, V - start);
    uint32_t klo = klo0, khi = khi0;
    if (!prescored || refill) score_split<MODE>(p, t, seq, start, len, L, gsp, klo, khi);
    if (!refill) {
      tl_stamp(p.tl, kTlIndexer, kTlScored);
      tl_clock(p.tl, kTlIndexer, kTlClockEnd);
    }

    if (!refill) {
      if (nsplit == 1) {
        const Kth kt = radix_kth(L.keys, len, K_eff, klo, khi, L);
        emit_sel(L.keys, len, kt.T, K_eff - kt.gt,
                 [&](int slot, int i, uint32_t k) {
                   if (slot < K_eff) {
                     p.out_idx[(size_t)t * p.K + slot] = start + i;
                     if (p.out_score) p.out_score[(size_t)t * p.K + slot] = key_to_float(k);
                   }
                 },
                 L);
        pad_output(p, t, K_eff);
        return false;
      }
      // candidates of this split: every key at or above a threshold chosen so that a little
      // more than the split's expected share e of the Top-K survives
      {
        const float e = (float)K_eff * (float)len / (float)V;
        int m = (int)ceilf(e + 4.f * sqrtf(e) + 4.f);
        const int hard = min(len, cap);
        m = min(m, hard);
        // The cut is the bin of the m-th key unless that bin is crowded.  With many splits the
        // merge's list is long and its passes cost more than ranking within the bin here, so
        // then every split cuts at the exact m-th key (measured: one 1M-position query, 512
        // splits, 68.0 -> 63.6 us; eight 64K-128K queries, 49-86 splits, no gain).
        const int soft = nsplit > 128 ? m : min(hard, 2 * m);
        KeyBlock<kSplitMax / NT> kb;
        kb.load(L.keys, len);
        uint32_t tau = 0u;
        int cnt = len;
        if (m < len) {
          const int sh = range_shift(khi - klo);
          const BinPick bp = block_rank_bin(kb, klo, khi - klo, sh, m, L);
          tau = klo + ((uint32_t)bp.d << sh);
          cnt = bp.above + bp.c;
          if (cnt > soft) {
            // cut at the exact m-th key, ranked within its bin when the bin holds at most 64
            // keys
            const Kth kt = sh == 0 ? Kth{tau, bp.above, bp.above + bp.c}
                           : bp.c <= 64 ? block_bin_kth(kb, tau, (1u << sh) - 1u, bp.above, bp.c, m, L)
                                        : block_kth(kb, m, klo, khi, L);
            tau = kt.ge <= hard ? kt.T : kt.T + 1u;   // too many equal keys: only those above
            cnt = kt.ge <= hard ? kt.ge : kt.gt;
          }
        }
        // this split's run of the candidate area
        cnt = min(cnt, cap);
        tl_stamp(p.tl, kTlIndexer, kTlCut);
        const size_t cb = ((size_t)t * p.nsplit_max + cur) * p.rs;
        block_emit(kb, tau, 0x7fffffff,
                   [&](int slot, int i, uint32_t k) {
                     if (slot < cnt) {
                       st_agent(p.cand_key + cb + slot, k);
                       st_agent(p.cand_pos + cb + slot, start + i);
                     }
                   },
                   L);
        if ((int)threadIdx.x < ((cnt + 3) & ~3) - cnt) st_agent(p.cand_key + cb + cnt + threadIdx.x, 0u);
        if (threadIdx.x == 0) {
          uint32_t* h = p.hdr + ((size_t)t * p.nsplit_max + cur) * kHdrWords;
          st_agent(h, (uint32_t)cnt);
          st_agent(h + 1, tau);
          st_agent(h + 3, max(tau, klo));
          st_agent(h + 4, khi);
        }
      }
      // arrival: the last split of this query to arrive merges
      tl_stamp(p.tl, kTlIndexer, kTlStoresIssued);
      if (phase == 3) return false;
      wait_all_memory();
      __syncthreads();
      tl_stamp(p.tl, kTlIndexer, kTlEmitted);
      if (threadIdx.x == 0)
        L.bcast[0] = add_agent(p.counters + t, 1u) == (uint32_t)(nsplit - 1);
      __syncthreads();
      tl_stamp(p.tl, kTlIndexer, kTlArrived);
      tl_put(p.tl, kTlIndexer, kTlLast, L.bcast[0] ? 1u : 0u);
      if (!L.bcast[0]) return false;
      if (phase == 1) return true;
      if (merge<MODE>(p, t, K_eff, nsplit, Lm, T, gt, enough)) return false;
      refill = true;
      cur = -1;
    } else {
      // exact local Top-min(len, K_eff) of a failing split replaces its run (at most cap)
      const int kk = min(len, K_eff);
      const Kth kt = radix_kth(L.keys, len, kk, klo, khi, L);
      uint32_t* h = p.hdr + ((size_t)t * p.nsplit_max + cur) * kHdrWords;
      const size_t cb = ((size_t)t * p.nsplit_max + cur) * p.rs;
      emit_sel(L.keys, len, kt.T, kk - kt.gt,
               [&](int slot, int i, uint32_t k) {
                 if (slot < kk) {
                   st_agent(p.cand_key + cb + slot, k);
                   st_agent(p.cand_pos + cb + slot, start + i);
                 }
               },
               L);
      if ((int)threadIdx.x < ((kk + 3) & ~3) - kk) st_agent(p.cand_key + cb + kk + threadIdx.x, 0u);
      if (threadIdx.x == 0) {
        st_agent(h, (uint32_t)kk);
        st_agent(h + 1, 0u);
        st_agent(h + 3, kt.T);
        st_agent(h + 4, khi);
      }
    }
    // Next failing split, judged against the threshold the merge found.
    const int nxt = next_failing(cur);
    if (nxt < 0) {
      merge<MODE>(p, t, K_eff, nsplit, Lm, T, gt, enough);   // certified
      return false;
    }
    cur = nxt;
  }
}

// Work item (tile b of kMqQ consecutive queries, split j).  When two or more of the tile's
// queries have a split j and all of those read one sequence, score_mq scores them together
// and each then takes the rest of its split's steps in turn from its own scores; otherwise
// (and for queries without split j, which only pad their output or return) every query takes
// the single-query path.
template <int MODE>
__device__ __forceinline__ void run_tile(const IndexerParams& p, int b, int j, const Lds& L,
                                         const Lds& Lm, uint32_t* keys_mq, uint32_t* range_mq) {
  const int split = p.split, start = j * split;
  int tq[kMqQ], lens[kMqQ];
  int nq = 0, seq = -1, lenmax = 0;
  bool same = true;
  for (int i = 0; i < kMqQ; ++i) {
    const int t = kMqQ * b + i;
    if (t >= p.T) break;
    const int V = min(p.q_vis[t], p.max_visible);
    if (V <= start) continue;                 // no split j (or nothing visible)
    const int s = p.q_seq[t];
    if (nq > 0 && s != seq) same = false;
    seq = s;
    tq[nq] = t;
    lens[nq] = min(split, V - start);
    lenmax = max(lenmax, lens[nq]);
    ++nq;
  }
  for (int i = nq; i < kMqQ; ++i) tq[i] = lens[i] = 0;
  if (same && nq >= 2) {
    uint32_t* const keys[kMqQ] = {L.keys, keys_mq, keys_mq + kSplitMax, keys_mq + 2 * kSplitMax};
    constexpr bool F8 = MODE >= 2, MXK = MODE == 3;
    if (p.L.bt) score_mq<F8, true, MXK>(p, tq, nq, seq, start, lenmax, lens, keys, L, range_mq);
    else score_mq<F8, false, MXK>(p, tq, nq, seq, start, lenmax, lens, keys, L, range_mq);
    // every query's selection and emission first: a merge (and its re-scoring) takes the
    // whole region, where the other queries' scores are.  The candidate stores of all of them
    // are drained once, then the queries arrive together.
    for (int i = 0; i < nq; ++i) {
      Lds Lq = L;
      Lq.keys = keys[i];
      run_item<MODE>(p, tq[i], j, Lq, Lm, true, range_mq[2 * i], range_mq[2 * i + 1], 3);
      __syncthreads();
    }
    wait_all_memory();
    __syncthreads();
    if (threadIdx.x == 0) {
      for (int i = 0; i < nq; ++i) {
        const int V = min(p.q_vis[tq[i]], p.max_visible);
        const int ns = (V + split - 1) / split;
        L.bcast[i] = ns > 1 && add_agent(p.counters + tq[i], 1u) == (uint32_t)(ns - 1);
      }
    }
    __syncthreads();
    bool must_merge[kMqQ];
    for (int i = 0; i < kMqQ; ++i) must_merge[i] = i < nq && L.bcast[i];
    __syncthreads();
    for (int i = 0; i < nq; ++i)
      if (must_merge[i]) {
        run_item<MODE>(p, tq[i], j, L, Lm, false, 0u, 0u, 2);
        __syncthreads();
      }
    for (int i = 0; i < kMqQ; ++i) {          // queries without split j
      const int t = kMqQ * b + i;
      if (t < p.T && min(p.q_vis[t], p.max_visible) <= start) {
        run_item<MODE>(p, t, j, L, Lm);
        __syncthreads();
      }
    }
    return;
  }
  for (int i = 0; i < kMqQ; ++i) {
    const int t = kMqQ * b + i;
    if (t < p.T) {
      run_item<MODE>(p, t, j, L, Lm);
      __syncthreads();
    }
  }
}

// The reference path (MODE 0) keeps its fp32 query in LDS and fits one workgroup per CU; the
// MFMA paths fit two.
// MXFP8 keys (MFMA path): the queries are quantized the same way, per head and group of 32
// dims, once per call, and their dequantized values (an e4m3 value times a power of two, exact
// in bf16 for scale bytes >= 3) go to p.q_mx, from which the scorers read them like a bf16
// query.  Four workgroups per query, each a quarter (16 heads x 128 dims): thread i takes dims
// 8 (i % 16) .. + 7 of head 16 b + i / 16 of quarter b, so a group of 32 dims is four
// consecutive lanes, which share its largest magnitude by lane exchange.
__global__ __launch_bounds__(NT) void mx_query_kernel(IndexerParams p) {
  static_assert(NT == 256, "a quarter of a query (16 heads x 128 dims) per workgroup");
  const int t = blockIdx.x >> 2;
  const size_t off = (size_t)t * (64 * 128) + (size_t)(blockIdx.x & 3) * (16 * 128) + 8 * threadIdx.x;
  const bf16x8 v = *(const bf16x8*)((const uint16_t*)p.q + off);
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf((float)v[e]));
  // the group's 32 values are lanes 4k .. 4k + 3 of the wave
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  const uint32_t sbyte = mx_scale_byte(amax);
  const float inv = mx_inv_scale(sbyte), sc = mx_scale_f32(sbyte);
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)(fp8_e4m3_to_f32(f32_to_fp8_e4m3_nb((float)v[e] * inv)) * sc);
  *(bf16x8*)(p.q_mx + off) = r;
}

template <int MODE, int QT = 1>
__global__ __launch_bounds__(NT, MODE == 0 ? 1 : 2) void indexer_topk_kernel(IndexerParams p) {
  constexpr int RB = region_bytes<MODE>();
  static_assert(RB >= kBins * 4 && flat_words<MODE>() >= kNSplitMax + 4, "shared region");
  __shared__ __attribute__((aligned(16))) uint8_t s_region[RB];
  __shared__ __attribute__((aligned(16))) uint32_t s_keys[kSplitMax];
  __shared__ __attribute__((aligned(16))) float s_w[NWAVE * 64];
  __shared__ int s_res[4], s_scan[2 * NWAVE + 2], s_wcnt[2 * NWAVE], s_bcast[4];
  __shared__ uint32_t s_range[2 * NWAVE];
  __shared__ __attribute__((aligned(16))) int s_psum[NT];
  __shared__ uint32_t s_small[64], s_small_w[64];
  Lds L;
  L.keys = s_keys;
  L.w = s_w;
  L.region = s_region;
  L.hist = (int*)s_region;                         // while selecting a split's candidates
  L.sel_key = (uint32_t*)s_region;                 // while merging (hist then moves to s_keys)
  L.sel_pos = (int32_t*)(s_region + kSelCap * 4);
  L.flat = (uint32_t*)(s_region + kSelBytes);
  L.res = s_res;
  L.scan = s_scan;
  L.wcnt = s_wcnt;
  L.bcast = s_bcast;
  L.range = s_range;
  L.psum = s_psum;
  L.small = s_small;
  L.small_w = s_small_w;
  Lds Lm = L;
  Lm.hist = (int*)s_keys;
  tl_stamp(p.tl, kTlIndexer, kTlStart);
  tl_clock(p.tl, kTlIndexer, kTlClockStart);
  if constexpr (QT > 1) {
    // one item (tile of QT queries, split j) per workgroup, j-major with the tiles rotated
    // by j as the queries are below
    static_assert(QT == kMqQ && QT == NWAVE && MODE >= 1, "multi-query tiles: MFMA paths");
    uint32_t* const s_keys_mq = (uint32_t*)(s_region + kMqKeysOff);
    __shared__ uint32_t s_range_mq[2 * QT];
    const int ntiles = (p.T + QT - 1) / QT;
    const int item = blockIdx.x;
    const int j = item / ntiles, b = (item - j * ntiles + j) % ntiles;
    run_tile<MODE>(p, b, j, L, Lm, s_keys_mq, s_range_mq);
    return;
  }

  // Work items (query t, split j).  Compact launch: the items, query-major, are numbered from
  // the queries' split counts, and workgroup i takes items i, i + grid, ... so that a grid
  // sized from the host's estimate covers every item even when the estimate is short.
  // Otherwise one item per workgroup by the linear index: the splits that exist for every
  // query (small j) come first and the empty ones of short queries last, so the live
  // workgroups spread over all the CUs, and within a block of T workgroups the queries are
  // rotated by j so that each query's splits spread over the XCDs.
  __shared__ int s_pre[kCompactMaxT + 1];
  int n_items = gridDim.x;
  if (p.compact) {
    if ((int)threadIdx.x < p.T) {
      const int V = min(p.q_vis[threadIdx.x], p.max_visible);
      s_pre[threadIdx.x + 1] = V <= 0 ? 1 : (V + p.split - 1) / p.split;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      s_pre[0] = 0;
      for (int u = 0; u < p.T; ++u) s_pre[u + 1] += s_pre[u];
    }
    __syncthreads();
    n_items = s_pre[p.T];
  }
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    int t, j;
    if (p.compact) {
      t = 0;
      while (s_pre[t + 1] <= item) ++t;
      j = item - s_pre[t];
    } else {
      j = item / p.T;
      t = (item - j * p.T + j) % p.T;
    }
    run_item<MODE>(p, t, j, L, Lm);
    __syncthreads();
  }
}

}  // namespace

// The build compiles this file once per part (DSA_INDEXER_PART = 0 .. 3) so that the kernel's
// instantiations compile in parallel; part 0 also holds the host planners and the dispatcher.
// Without the macro every part is in one translation unit.
#ifndef DSA_INDEXER_PART
#define DSA_INDEXER_PART -1
#endif
#define DSA_PART(n) (DSA_INDEXER_PART < 0 || DSA_INDEXER_PART == (n))

template <int MODE, int QT>
void launch_instance(dim3 grid, hipStream_t stream, const IndexerParams& p);
#define DSA_INSTANCE(part, MODE, QT)                                                         \
  template <>                                                                                \
  void launch_instance<MODE, QT>(dim3 grid, hipStream_t stream, const IndexerParams& p) {    \
    hipLaunchKernelGGL((indexer_topk_kernel<MODE, QT>), grid, dim3(NT), 0, stream, p);       \
  }
#if DSA_PART(0)
DSA_INSTANCE(0, 0, 1)
DSA_INSTANCE(0, 1, 1)
#endif
#if DSA_PART(1)
DSA_INSTANCE(1, 2, 1)
DSA_INSTANCE(1, 1, kMqQ)
#endif
#if DSA_PART(2)
DSA_INSTANCE(2, 3, 1)
DSA_INSTANCE(2, 2, kMqQ)
#endif
#if DSA_PART(3)
DSA_INSTANCE(3, 3, kMqQ)
#endif

#if DSA_PART(0)
// The layout and launch for one split length (a multiple of 64 in [kMinSplit, kSplitMax]).
IndexerPlan plan_indexer_split(int32_t T, int32_t max_visible, int32_t top_k, int32_t split) {
  IndexerPlan pl{};
  pl.split = split;
  pl.nsplit_max = (int32_t)((max_visible + split - 1) / split);
  pl.cap = (int32_t)(split < top_k ? split : top_k);
  pl.rs = (pl.cap + 3) / 4 * 4;
  pl.grid = pl.nsplit_max * T;
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  // one run of rs candidate slots per split
  const size_t slots = (size_t)T * pl.nsplit_max * pl.rs;
  size_t off = 0;
  pl.off_counters = 0;
  off = al((size_t)T * 4);
  if (off < kCtrlBytes) off = kCtrlBytes;
  pl.off_hdr = off;      off = al(off + (size_t)T * pl.nsplit_max * 32);
  pl.off_ckey = off;     off = al(off + slots * 4);
  pl.off_cpos = off;     off = al(off + slots * 4);
  // MXFP8 keys on the MFMA path: every query quantized once per call (64 x 128 bf16 values)
  pl.off_qmx = off;      off = al(off + (size_t)T * 64 * 128 * 2);
  pl.bytes = off;
  return pl;
}

// Split length: the live workgroups (sum over queries of ceil(V_t / split)) should fill the
// chip's 512 resident slots (256 CUs x 2) without exceeding them; a workgroup that has to wait
// for a slot starts only when another ends and delays its query's merge by a whole split.
// With the total visible length known, split = total / (512 - T) bounds the live count by
// 512; without it, T * max_visible stands in for the total (fewer, longer splits).
IndexerPlan plan_indexer(int32_t T, int32_t max_visible, int32_t top_k, int64_t total_visible) {
  const int64_t target_wg = plan_overrides().indexer_target_wg > 0 ? plan_overrides().indexer_target_wg : 512;
  const int64_t tmax = (int64_t)T * max_visible;
  int64_t total = tmax, slots = target_wg;
  if (total_visible > 0) {
    total = total_visible < max_visible ? max_visible : (total_visible > tmax ? tmax : total_visible);
    if (T < target_wg / 2) slots = target_wg - T;
  }
  int64_t split = (total + slots - 1) / slots;
  split = (split + 63) / 64 * 64;
  if (split < kMinSplit) split = kMinSplit;
  if (split > kSplitMax) split = kSplitMax;
  IndexerPlan pl = plan_indexer_split(T, max_visible, top_k, (int32_t)split);
  if (total_visible > 0 && T <= kCompactMaxT) {
    // no empty workgroups: at most total / split + T items exist (one partial split a query)
    const int64_t items = (total + split - 1) / split + T;
    pl.compact = 1;
    if (items < pl.grid) pl.grid = (int32_t)items;
  }
  return pl;
}

// Workspace large enough for every split length a plan can choose.
size_t indexer_workspace_bytes(int32_t T, int32_t max_visible, int32_t top_k) {
  size_t b = 0;
  for (int32_t s = kMinSplit; s <= kSplitMax; s += 64) {
    const size_t x = plan_indexer_split(T, max_visible, top_k, s).bytes;
    b = x > b ? x : b;
  }
  return b;
}

// Multi-query tiles for many queries on the MFMA paths (chunked prefill: thousands of queries
// over one cached context); DSA_INDEXER_MQ=0 turns them off for measurement.
bool indexer_multi_query(const IndexerParams& p) {
  if (p.compact || p.T < kMqMinT) return false;
  return !plan_overrides().indexer_mq_off;
}

hipError_t launch_indexer(const IndexerParams& p, bool fast_path, hipStream_t stream) {
  const dim3 grid(p.grid);
  const bool mq = fast_path && indexer_multi_query(p);
  const dim3 gmq(p.nsplit_max * ((p.T + kMqQ - 1) / kMqQ));
  if (fast_path && p.k_dtype == kDtMX) {
    // the queries' MXFP8 quantization, once per call, ahead of the scoring
    hipLaunchKernelGGL(mx_query_kernel, dim3(4 * p.T), dim3(NT), 0, stream, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!fast_path) launch_instance<0, 1>(grid, stream, p);
  else if (p.k_dtype == kDtFP8) mq ? launch_instance<2, kMqQ>(gmq, stream, p) : launch_instance<2, 1>(grid, stream, p);
  else if (p.k_dtype == kDtMX) mq ? launch_instance<3, kMqQ>(gmq, stream, p) : launch_instance<3, 1>(grid, stream, p);
  else mq ? launch_instance<1, kMqQ>(gmq, stream, p) : launch_instance<1, 1>(grid, stream, p);
  return hipGetLastError();
}
#endif  // DSA_PART(0)

}  // namespace dsa
