// Sparse Flash Attention over selected rows of the paged MLA latent cache (gfx950).
//
// For query t and head h:  z_j = scale * q[t,h,:] . R_j,  out[t,h,:] = softmax(z) . R[:, :d_v],
// where R_j is the 576-wide latent row of the j-th selected position and its first 512
// columns are the value.  SFA reads the main KV only at the indexer's positions ("Day0
// Adaptation and Performance Optimization for Novel Long-Sequence Reasoning Models",
// section 3); the rows are fetched a whole row at a time with 16-byte vector loads, the
// block-wise vectorized sparse reads of "Day0 Adaptation and Sparse Attention Optimization
// for Long-Sequence LLM Inference", section 4.
//
// Fast path (bf16 storage, d_qk = 576, d_v = 512): a workgroup owns (query, group of 16*NW
// heads, slice of the index list).  Per tile of 32 selected rows it gathers the rows into LDS
// twice: row-major for Q.K^T and transposed (dims x rows) for P.V, so both contractions
// read 16-byte MFMA operands from LDS.  Each wave holds 16 heads: their queries stay in
// registers (B operand), S^T = R . Q^T comes out of v_mfma_f32_16x16x32_bf16 with one head per
// lane column, online softmax runs in the exp2 domain, and the probabilities in that same
// lane layout are the A operand of the P.V MFMA (the row order of the transposed tile is
// permuted to match).  O accumulates in fp32.  Slices of the index list are merged by a
// log-sum-exp weighted combine kernel.
// Reference path (fp32 storage or other shapes): one workgroup per (query, head), fp32.

#include "dsa_internal.hpp"

namespace dsa {
namespace {

constexpr int kTileRows = 32;
constexpr int kRowBytes = kSfaDqk * 2;            // 1152
constexpr int kKvStride = kRowBytes + 16;         // padded LDS row
constexpr int kVtStride = kTileRows * 2 + 16;     // padded LDS dim-row of the transposed tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// slot of tile row r in the transposed tile: k-slice 8g..8g+7 of the P.V MFMA holds rows
// 4g..4g+3 and 16+4g..16+4g+3, the rows one lane owns in the S^T accumulator layout.
__device__ __forceinline__ int vt_slot(int r) {
  return r < 16 ? 8 * (r >> 2) + (r & 3) : 8 * ((r - 16) >> 2) + 4 + ((r - 16) & 3);
}

template <int NW>
__global__ __launch_bounds__(NW * 64) void sfa_mfma_kernel(SfaParams p) {
  constexpr int NTS = NW * 64;
  __shared__ __attribute__((aligned(16))) uint8_t kv_lds[kTileRows * kKvStride];
  __shared__ __attribute__((aligned(16))) uint8_t vt_lds[kSfaDv * kVtStride];
  __shared__ int64_t rows[kTileRows];

  const int r = blockIdx.x, hg = blockIdx.y, t = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int h0 = hg * p.heads_per_wg + wave * 16;
  const int seq = p.q_seq[t];

  // queries of this wave's 16 heads: lane holds head c16, dims 32s + 8g .. +7
  bf16x8 qr[18];
  {
    const uint16_t* qb = (const uint16_t*)p.q + ((size_t)t * p.H + h0 + c16) * kSfaDqk + 8 * g;
#pragma unroll
    for (int s = 0; s < 18; ++s) qr[s] = *(const bf16x8*)(qb + 32 * s);
  }
  const float scale2 = p.scale * kLog2e;
  float m2 = -INFINITY, l = 0.f;
  f32x4 o[32];
#pragma unroll
  for (int n = 0; n < 32; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int j0 = r * p.rows_per_split;
  const int j1 = min(p.K, j0 + p.rows_per_split);
  const int32_t* idx = p.idx + (size_t)t * p.K;
  const uint8_t* kv = (const uint8_t*)p.kv;

  for (int tile = j0; tile < j1; tile += kTileRows) {
    __syncthreads();
    if (tid < kTileRows) {
      const int jj = tile + tid;
      const int pos = jj < j1 ? idx[jj] : -1;
      rows[tid] = pos >= 0 ? pool_row(p.L, seq, pos) : (int64_t)-1;
    }
    __syncthreads();
    for (int c = tid; c < kTileRows * 72; c += NTS) {
      const int rr = c / 72, cc = c - rr * 72;
      const int64_t pr = rows[rr];
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (pr >= 0) v = __builtin_nontemporal_load((const u32x4*)(kv + pr * kRowBytes) + cc);
      *(u32x4*)(kv_lds + rr * kKvStride + cc * 16) = v;
      if (cc < 64) {
        const int slot = vt_slot(rr);
        const uint32_t e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const uint16_t h = (uint16_t)(e[u >> 1] >> (16 * (u & 1)));
          *(uint16_t*)(vt_lds + (8 * cc + u) * kVtStride + 2 * slot) = h;
        }
      }
    }
    __syncthreads();

    // S^T = R . Q^T for tile rows 0..15 and 16..31
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    const uint8_t* ra = kv_lds + c16 * kKvStride + 16 * g;
    const uint8_t* rb = kv_lds + (16 + c16) * kKvStride + 16 * g;
#pragma unroll
    for (int s = 0; s < 18; ++s) {
      const bf16x8 a0 = *(const bf16x8*)(ra + 64 * s);
      const bf16x8 a1 = *(const bf16x8*)(rb + 64 * s);
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qr[s], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qr[s], s1, 0, 0, 0);
    }
    float z[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      z[i] = rows[4 * g + i] >= 0 ? s0[i] * scale2 : -INFINITY;
      z[4 + i] = rows[16 + 4 * g + i] >= 0 ? s1[i] * scale2 : -INFINITY;
    }
    float mx = z[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mx = fmaxf(mx, z[i]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mn = fmaxf(m2, mx);
    const bool live = mn != -INFINITY;
    const float alpha = live ? exp2f(m2 - mn) : 1.f;
    float pr8[8], ps = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pr8[i] = live ? exp2f(z[i] - mn) : 0.f;
      ps += pr8[i];
    }
    l = l * alpha + ps;
    m2 = mn;
    // O rows held by this lane are heads 4g..4g+3: their rescale factors live in lanes 4g+i
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float ai = __shfl(alpha, 4 * g + i, 64);
#pragma unroll
      for (int n = 0; n < 32; ++n) o[n][i] *= ai;
    }
    bf16x8 pa;
#pragma unroll
    for (int i = 0; i < 8; ++i) pa[i] = (__bf16)pr8[i];
    const uint8_t* vb = vt_lds + c16 * kVtStride + 16 * g;
#pragma unroll
    for (int n = 0; n < 32; ++n) {
      const bf16x8 b = *(const bf16x8*)(vb + 16 * n * kVtStride);
      o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, b, o[n], 0, 0, 0);
    }
  }

  // per-head totals: lanes sharing c16 hold disjoint rows of the same head
  float lt = l + __shfl_xor(l, 16, 64);
  lt += __shfl_xor(lt, 32, 64);
  float lrow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) lrow[i] = __shfl(lt, 4 * g + i, 64);

  if (p.nsplit == 1) {
    uint16_t* out = (uint16_t*)p.out + ((size_t)t * p.H + h0) * kSfaDv;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float inv = lrow[i] > 0.f ? 1.f / lrow[i] : 0.f;
#pragma unroll
      for (int n = 0; n < 32; ++n)
        out[(4 * g + i) * kSfaDv + 16 * n + c16] = (uint16_t)f32_to_bf16_bits(o[n][i] * inv);
    }
    if (p.lse && g == 0)
      p.lse[(size_t)t * p.H + h0 + c16] = lt > 0.f ? (m2 + log2f(lt)) * kLn2 : -INFINITY;
  } else {
    const size_t pb = (((size_t)t * p.H + h0) * p.nsplit + r);   // (t, head h0, split r)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float* po = p.part_o + (pb + (size_t)(4 * g + i) * p.nsplit) * kSfaDv;
#pragma unroll
      for (int n = 0; n < 32; ++n) po[16 * n + c16] = o[n][i];
    }
    if (g == 0) {
      float* pm = p.part_ml + (pb + (size_t)c16 * p.nsplit) * 2;
      pm[0] = m2;
      pm[1] = lt;
    }
  }
}

// Log-sum-exp weighted merge of the index-list slices: one workgroup per (query, 16 heads).
__global__ __launch_bounds__(256) void sfa_combine_kernel(SfaParams p) {
  __shared__ float wts[16][64];
  __shared__ float lse_s[16];
  const int hb = blockIdx.x * 16, t = blockIdx.y;
  const int ns = p.nsplit;
  if (threadIdx.x < 16) {
    const int h = hb + threadIdx.x;
    const float* pm = p.part_ml + (((size_t)t * p.H + h) * ns) * 2;
    float M = -INFINITY;
    for (int r = 0; r < ns; ++r) M = fmaxf(M, pm[2 * r]);
    float L = 0.f;
    for (int r = 0; r < ns; ++r) {
      const float w = M == -INFINITY ? 0.f : exp2f(pm[2 * r] - M) * pm[2 * r + 1];
      L += w;
    }
    for (int r = 0; r < ns; ++r)
      wts[threadIdx.x][r] = (L > 0.f) ? exp2f(pm[2 * r] - M) / L : 0.f;
    lse_s[threadIdx.x] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 16 * kSfaDv; e += 256) {
    const int hh = e / kSfaDv, d = e - hh * kSfaDv;
    const float* po = p.part_o + (((size_t)t * p.H + hb + hh) * ns) * kSfaDv + d;
    float acc = 0.f;
    for (int r = 0; r < ns; ++r) acc += wts[hh][r] * po[(size_t)r * kSfaDv];
    ((uint16_t*)p.out)[((size_t)t * p.H + hb + hh) * kSfaDv + d] = (uint16_t)f32_to_bf16_bits(acc);
  }
  if (p.lse && threadIdx.x < 16) p.lse[(size_t)t * p.H + hb + threadIdx.x] = lse_s[threadIdx.x];
}

// Reference mode: one workgroup per (query, head), fp32 everywhere.
constexpr int kRefThreads = 256;
__global__ __launch_bounds__(kRefThreads) void sfa_reference_kernel(SfaParams p) {
  __shared__ float qs[1024];
  __shared__ float z[2048];
  __shared__ int64_t rws[2048];
  __shared__ float red[kRefThreads / 64];
  const int h = blockIdx.x, t = blockIdx.y;
  const int tid = threadIdx.x;
  const int seq = p.q_seq[t];
  const bool f32 = p.dtype == kDtF32;
  for (int d = tid; d < p.dqk; d += kRefThreads) {
    const size_t qi = ((size_t)t * p.H + h) * p.dqk + d;
    qs[d] = f32 ? ((const float*)p.q)[qi] : bf16_bits_to_f32(((const uint16_t*)p.q)[qi]);
  }
  __syncthreads();
  auto kvat = [&](int64_t row, int d) -> float {
    const size_t i = (size_t)row * p.dqk + d;
    return f32 ? ((const float*)p.kv)[i] : bf16_bits_to_f32(((const uint16_t*)p.kv)[i]);
  };
  float lmax = -INFINITY;
  for (int j = tid; j < p.K; j += kRefThreads) {
    const int pos = p.idx[(size_t)t * p.K + j];
    float zz = -INFINITY;
    int64_t row = -1;
    if (pos >= 0) {
      row = pool_row(p.L, seq, pos);
      float acc = 0.f;
      for (int d = 0; d < p.dqk; ++d) acc = fmaf(qs[d], kvat(row, d), acc);
      zz = acc * p.scale;
    }
    z[j] = zz;
    rws[j] = row;
    lmax = fmaxf(lmax, zz);
  }
  // block max
  for (int off = 32; off >= 1; off >>= 1) lmax = fmaxf(lmax, __shfl_xor(lmax, off, 64));
  if ((tid & 63) == 0) red[tid >> 6] = lmax;
  __syncthreads();
  float M = red[0];
  for (int w = 1; w < kRefThreads / 64; ++w) M = fmaxf(M, red[w]);
  __syncthreads();
  float ls = 0.f;
  for (int j = tid; j < p.K; j += kRefThreads) {
    const float e = (M == -INFINITY || rws[j] < 0) ? 0.f : expf(z[j] - M);
    z[j] = e;
    ls += e;
  }
  for (int off = 32; off >= 1; off >>= 1) ls += __shfl_xor(ls, off, 64);
  if ((tid & 63) == 0) red[tid >> 6] = ls;
  __syncthreads();
  float L = 0.f;
  for (int w = 0; w < kRefThreads / 64; ++w) L += red[w];
  const float inv = L > 0.f ? 1.f / L : 0.f;
  for (int d = tid; d < p.dv; d += kRefThreads) {
    float acc = 0.f;
    for (int j = 0; j < p.K; ++j)
      if (rws[j] >= 0) acc = fmaf(z[j], kvat(rws[j], d), acc);
    const size_t oi = ((size_t)t * p.H + h) * p.dv + d;
    if (f32) ((float*)p.out)[oi] = acc * inv;
    else ((uint16_t*)p.out)[oi] = (uint16_t)f32_to_bf16_bits(acc * inv);
  }
  if (p.lse && tid == 0) p.lse[(size_t)t * p.H + h] = L > 0.f ? M + logf(L) : -INFINITY;
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
    pl.heads_per_wg = (H % 64 == 0) ? 64 : (H % 32 == 0) ? 32 : 16;
    pl.n_hg = H / pl.heads_per_wg;
    const int64_t want = 512;
    int64_t ns = (want + (int64_t)T * pl.n_hg - 1) / ((int64_t)T * pl.n_hg);
    const int64_t max_ns = (K + kTileRows - 1) / kTileRows;
    if (ns < 1) ns = 1;
    if (ns > max_ns) ns = max_ns;
    int64_t rps = (K + ns - 1) / ns;
    rps = (rps + kTileRows - 1) / kTileRows * kTileRows;
    pl.rows_per_split = (int32_t)rps;
    pl.nsplit = (int32_t)((K + rps - 1) / rps);
  }
  size_t off = 0;
  pl.off_counters = off;
  off = al(off + 16);
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
  const dim3 grid(p.nsplit, p.n_hg, p.T);
  switch (p.heads_per_wg) {
    case 64: hipLaunchKernelGGL(sfa_mfma_kernel<4>, grid, dim3(256), 0, stream, p); break;
    case 32: hipLaunchKernelGGL(sfa_mfma_kernel<2>, grid, dim3(128), 0, stream, p); break;
    default: hipLaunchKernelGGL(sfa_mfma_kernel<1>, grid, dim3(64), 0, stream, p); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.nsplit == 1) return e;
  hipLaunchKernelGGL(sfa_combine_kernel, dim3(p.H / 16, p.T), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace dsa
