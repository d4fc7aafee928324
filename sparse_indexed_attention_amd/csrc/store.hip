// Cache writers: place new tokens into the paged pools in the layout the indexer and SFA read.
//
// Index keys may be stored in fp8-e4m3 with one fp32 scale per token, the quantized indexer
// path of "Day0 Adaptation and Performance Optimization for Novel Long-Sequence Reasoning
// Models", section 3 (the pages' group-32 MXFP8 variant is not this format): scale =
// max|k| / 448 (1 for an all-zero token), code = e4m3(k / scale) rounded to nearest even and
// saturated at +-448.  One wave per token.

#include "dsa_internal.hpp"

namespace dsa {
namespace {

// fp32 -> e4m3fn code, nearest value with ties to the even code, |x| >= 448 -> 448, NaN ->
// 0x7F.  Within one binade the e4m3 values are evenly spaced and the code's low bit is the
// mantissa's, so rounding the scaled mantissa to the nearest even integer is exactly "ties to
// the even code"; a carry into the next binade lands on mantissa 0, also even.
__device__ __forceinline__ uint32_t f32_to_fp8_e4m3(float x) {
  if (x != x) return 0x7fu;
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fabsf(x);
  if (a >= 448.f) return sign | 0x7eu;
  if (a < 0.015625f) {                                   // below 2^-6: subnormal grid m*2^-9
    const uint32_t n = (uint32_t)rintf(a * 512.f);       // exact scaling, then RNE; n <= 8
    return sign | n;                                     // n == 8 is code 0x08 = 2^-6
  }
  int E = (int)((__float_as_uint(a) >> 23) & 0xffu) - 127;   // -6 .. 8
  const float m = a * __uint_as_float((uint32_t)(127 - E) << 23);   // a / 2^E, exact, in [1,2)
  uint32_t n = (uint32_t)rintf((m - 1.f) * 8.f);
  if (n == 8u) { n = 0u; ++E; }
  return sign | ((uint32_t)(E + 7) << 3) | n;
}

__global__ __launch_bounds__(64) void store_index_keys_kernel(const float* k_new, int D,
                                                              const int64_t* slot, void* pool,
                                                              int dt, float* k_scale) {
  const int i = blockIdx.x, lane = threadIdx.x;
  const float* src = k_new + (size_t)i * D;
  const int64_t row = slot[i];
  if (dt == kDtF32) {
    for (int d = lane; d < D; d += 64) ((float*)pool)[row * D + d] = src[d];
    return;
  }
  if (dt == kDtBF16) {
    for (int d = lane; d < D; d += 64)
      ((uint16_t*)pool)[row * D + d] = (uint16_t)f32_to_bf16_bits(src[d]);
    return;
  }
  float amax = 0.f;
  for (int d = lane; d < D; d += 64) amax = fmaxf(amax, fabsf(src[d]));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  const float scale = amax == 0.f ? 1.f : amax / 448.f;
  for (int d = lane; d < D; d += 64)
    ((uint8_t*)pool)[row * D + d] = (uint8_t)f32_to_fp8_e4m3(src[d] / scale);
  if (lane == 0) k_scale[row] = scale;
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

}  // namespace

hipError_t launch_store_index_keys(const float* k_new, int32_t n, int32_t D, const int64_t* slot,
                                   void* k_pool, int32_t k_dtype, float* k_scale, hipStream_t s) {
  hipLaunchKernelGGL(store_index_keys_kernel, dim3(n), dim3(64), 0, s, k_new, D, slot, k_pool,
                     k_dtype, k_scale);
  return hipGetLastError();
}

hipError_t launch_store_kv(const void* kv_new, int32_t src_dtype, int32_t n, int32_t dqk,
                           const int64_t* slot, void* kv_pool, int32_t pool_dtype, hipStream_t s) {
  hipLaunchKernelGGL(store_kv_kernel, dim3(n), dim3(256), 0, s, kv_new, src_dtype, dqk, slot,
                     kv_pool, pool_dtype);
  return hipGetLastError();
}

}  // namespace dsa
