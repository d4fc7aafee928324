// One index-key row written into the key pool in its storage format, by one wave (64 lanes).
// The formats are those of dsa_store_index_keys: f32; bf16 (nearest even); fp8-e4m3 with one
// fp32 scale per token (max |k| / 448, 1 for an all-zero token); MXFP8 (per group of 32 dims
// an E8M0 byte, see mx_scale_byte, and e4m3 codes of k * 2^(127 - byte)).  src may be in
// global memory or LDS.
#pragma once
#include "dsa_internal.hpp"

namespace dsa {

__device__ __forceinline__ void store_key_row(const float* src, int D, int64_t row, void* pool,
                                              int dt, float* k_scale, int lane) {
  if (dt == kDtF32) {
    for (int d = lane; d < D; d += 64) ((float*)pool)[row * D + d] = src[d];
    return;
  }
  if (dt == kDtBF16) {
    for (int d = lane; d < D; d += 64)
      ((uint16_t*)pool)[row * D + d] = (uint16_t)f32_to_bf16_bits(src[d]);
    return;
  }
  if (dt == kDtMX) {
    // column d = d0 + lane: lanes 0..31 and 32..63 each hold one group of 32 (D % 32 == 0)
    uint8_t* sbytes = (uint8_t*)k_scale + row * (D / 32);
    for (int d0 = 0; d0 < D; d0 += 64) {
      const int d = d0 + lane;
      const float x = d < D ? src[d] : 0.f;
      float amax = fabsf(x);
#pragma unroll
      for (int off = 16; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
      const uint32_t sb = mx_scale_byte(amax);
      if (d < D) {
        ((uint8_t*)pool)[row * D + d] = (uint8_t)f32_to_fp8_e4m3(x * mx_inv_scale(sb));
        if ((lane & 31) == 0) sbytes[d >> 5] = (uint8_t)sb;
      }
    }
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

}  // namespace dsa
