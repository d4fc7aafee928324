// Cache writers: place new tokens into the paged pools in the layout the indexer and SFA read.
//
// Index keys may be stored in fp8-e4m3 with one fp32 scale per token, the quantized indexer
// path of "Day0 Adaptation and Performance Optimization for Novel Long-Sequence Reasoning
// Models", section 3 (the pages' group-32 MXFP8 variant is not this format): scale =
// max|k| / 448 (1 for an all-zero token), code = e4m3(k / scale) rounded to nearest even and
// saturated at +-448.  One wave per token.
//
// Index keys may also be stored in MXFP8 ("Day0 Adaptation and Performance Optimization for
// Novel Long-Sequence Reasoning Models", section 4; "Optimizing and Deploying Ultra-Long
// Sequence Inference Architectures", section II: groups of 32 elements share one scale), read
// as the OCP microscaling format: per group of 32 dims an E8M0 byte (see mx_scale_byte) and
// e4m3 codes of k * 2^(127 - byte), nearest even, saturated.
//
// The SFA latent cache may be stored in fp8-e4m3 per token and per tile of 128 columns ("Day0
// Adaptation and Performance Optimization for Novel Long-Sequence Reasoning Models", section
// 4; "Large Model Inference Acceleration: Day-0 Adaptation...", section 2.2): columns 0..511
// in four tiles, each with the smallest power-of-two scale 2^e that keeps the tile's largest
// magnitude at or below 448 (so no code saturates and x / scale is exact), the rope columns
// 512..575 in bf16.  One workgroup of 128 threads per token, thread i owning columns 4i..4i+3.

#include "store_row.hpp"

namespace dsa {
namespace {

__global__ __launch_bounds__(64) void store_index_keys_kernel(const float* k_new, int D,
                                                              const int64_t* slot, void* pool,
                                                              int dt, float* k_scale) {
  const int i = blockIdx.x;
  store_key_row(k_new + (size_t)i * D, D, slot[i], pool, dt, k_scale, threadIdx.x);
}

__global__ __launch_bounds__(256) void store_kv_kernel(const void* src, int sdt, int dqk,
                                                       const int64_t* slot, void* pool, int pdt) {
  const int i = blockIdx.x;
  const int64_t row = slot[i];
  for (int d = threadIdx.x; d < dqk; d += 256) {
    const size_t si = (size_t)i * dqk + d;
    const float v = sdt == kDtF32 ? ((const float*)src)[si]
                                  : bf16_bits_to_f32(((const uint16_t*)src)[si]);
    const int64_t di = row * dqk + d;
    if (pdt == kDtF32) ((float*)pool)[di] = v;
    else if (sdt == kDtBF16) ((uint16_t*)pool)[di] = ((const uint16_t*)src)[si];
    else ((uint16_t*)pool)[di] = (uint16_t)f32_to_bf16_bits(v);
  }
}

// Smallest power of two 2^e (-126 <= e) with amax <= 448 * 2^e; 1 for amax == 0.  With
// amax = m * 2^k (1 <= m < 2): 448 = 1.75 * 2^8, so e = k - 8, or k - 7 when m > 1.75.
__device__ __forceinline__ float tile_scale(float amax) {
  if (amax == 0.f) return 1.f;
  const uint32_t b = __float_as_uint(amax);
  const int be = (int)(b >> 23);                          // biased exponent (0: subnormal)
  int e = be == 0 ? -126 : be - 127 - 8 + ((b & 0x7fffffu) > 0x600000u ? 1 : 0);
  e = max(e, -126);
  return __uint_as_float((uint32_t)(e + 127) << 23);
}

__global__ __launch_bounds__(128) void store_kv_fp8_kernel(const void* src, int sdt,
                                                           const int64_t* slot, uint8_t* pool) {
  const int i = blockIdx.x, tid = threadIdx.x;
  uint8_t* dst = pool + slot[i] * (int64_t)kSfaRowF8;
  float x[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const size_t si = (size_t)i * kSfaDqk + 4 * tid + u;
    x[u] = sdt == kDtF32 ? ((const float*)src)[si] : bf16_bits_to_f32(((const uint16_t*)src)[si]);
  }
  // the tile of these columns is threads 32 (tid / 32) .. +31: a 32-lane reduction
  float amax = fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3])));
#pragma unroll
  for (int off = 16; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  const float scale = tile_scale(amax);
  uint32_t packed = 0u;
#pragma unroll
  for (int u = 0; u < 4; ++u) packed |= f32_to_fp8_e4m3(x[u] / scale) << (8 * u);
  *(uint32_t*)(dst + 4 * tid) = packed;
  if ((tid & 31) == 0) *(float*)(dst + 640 + 4 * (tid >> 5)) = scale;
  if (tid < 32) {
    // rope columns 512 + 2 tid, +1
    uint32_t w = 0u;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const size_t si = (size_t)i * kSfaDqk + kSfaDv + 2 * tid + u;
      const uint32_t bits = sdt == kDtF32 ? (uint32_t)f32_to_bf16_bits(((const float*)src)[si])
                                          : (uint32_t)((const uint16_t*)src)[si];
      w |= bits << (16 * u);
    }
    *(uint32_t*)(dst + 512 + 4 * tid) = w;
  }
}

}  // namespace

hipError_t launch_store_index_keys(const float* k_new, int32_t n, int32_t D, const int64_t* slot,
                                   void* k_pool, int32_t k_dtype, float* k_scale, hipStream_t s) {
  hipLaunchKernelGGL(store_index_keys_kernel, dim3(n), dim3(64), 0, s, k_new, D, slot, k_pool,
                     k_dtype, k_scale);
  return hipGetLastError();
}

hipError_t launch_store_kv(const void* kv_new, int32_t src_dtype, int32_t n, int32_t dqk,
                           const int64_t* slot, void* kv_pool, int32_t pool_dtype, hipStream_t s) {
  if (pool_dtype == kDtFP8) {
    hipLaunchKernelGGL(store_kv_fp8_kernel, dim3(n), dim3(128), 0, s, kv_new, src_dtype, slot,
                       (uint8_t*)kv_pool);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(store_kv_kernel, dim3(n), dim3(256), 0, s, kv_new, src_dtype, dqk, slot,
                     kv_pool, pool_dtype);
  return hipGetLastError();
}

}  // namespace dsa
