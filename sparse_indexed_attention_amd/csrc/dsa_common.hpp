// Device helpers shared by the DSA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// ---- scalar conversions ---------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) & 0x8000u) | 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// OCP e4m3fn code -> value (exact in fp32 / fp64).  Field layout: s.eeee.mmm, bias 7,
// exponent field 0 = subnormal m * 2^-9, s.1111.111 = NaN.
__device__ __forceinline__ float fp8_e4m3_to_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float v;
  if (e == 15u && m == 7u) v = __uint_as_float(0x7fc00000u);
  else if (e == 0u) v = (float)m * 0.001953125f;                       // m * 2^-9
  else v = __uint_as_float(((e + 120u) << 23) | (m << 20));            // 2^(e-7) * 1.m
  return (c & 0x80u) ? -v : v;
}

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

// The same code as f32_to_fp8_e4m3 for non-NaN x, without branches: with E = max(floor(log2
// |x|), -6) the e4m3 grid around |x| has spacing 2^(E-3) (the subnormal grid m * 2^-9 is the
// E = -6 case), so n = rint(|x| * 2^(3-E)) is the nearest grid point (ties to even n, i.e.
// to the even code); n = 16 carries into the next binade.  |x| is clamped to 448 first.
__device__ __forceinline__ uint32_t f32_to_fp8_e4m3_nb(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fminf(fabsf(x), 448.f);
  const int E = max((int)((__float_as_uint(a) >> 23) & 0xffu) - 127, -6);
  const uint32_t n = (uint32_t)rintf(a * __uint_as_float((uint32_t)(130 - E) << 23));   // a * 2^(3-E)
  const bool carry = n == 16u;
  const int Ef = carry ? E + 1 : E;
  const uint32_t nf = carry ? 8u : n;
  const uint32_t code = nf < 8u ? nf : ((uint32_t)(Ef + 7) << 3) | (nf - 8u);
  return sign | code;
}

// OCP microscaling (MX) E8M0 scale byte of a group of fp8-e4m3 elements: floor(log2(amax))
// minus 8 (the exponent of e4m3's largest power of two, 256), biased by 127 and clamped to
// [0, 254]; 0 for amax == 0.  The group's codes are e4m3(x * 2^(127 - byte)).
__device__ __forceinline__ uint32_t mx_scale_byte(float amax) {
  if (amax == 0.f) return 0u;
  const uint32_t b = __float_as_uint(amax);
  const int be = (int)(b >> 23);
  // floor(log2(amax)): the unbiased exponent, or for a subnormal the top set mantissa bit
  const int fl = be != 0 ? be - 127 : (31 - __clz((int)(b & 0x7fffffu))) - 149;
  return (uint32_t)min(max(fl - 8 + 127, 0), 254);
}
// 2^(byte - 127) as fp32 (byte 0: the subnormal 2^-127)
__device__ __forceinline__ float mx_scale_f32(uint32_t byte) {
  return __uint_as_float(byte ? byte << 23 : 0x00400000u);
}
// 2^(127 - byte) as fp32 (byte in [0, 254]: a normal number)
__device__ __forceinline__ float mx_inv_scale(uint32_t byte) {
  return __uint_as_float((254u - byte) << 23);
}

// Order-preserving map from fp32 to uint32: a larger float gives a larger key; -0 and +0
// give the same key.  NaN inputs are outside the contract.
__device__ __forceinline__ uint32_t float_to_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_to_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// ---- paged addressing -------------------------------------------------------------------
struct Layout {
  const int32_t* bt;      // block table or nullptr
  int32_t bt_stride;      // max_blocks_per_seq
  int32_t bs_log2;        // log2(block_size) when bt != nullptr
  int64_t seq_stride;     // rows between sequences when bt == nullptr
};

__device__ __forceinline__ int64_t pool_row(const Layout& L, int seq, int pos) {
  if (L.bt) {
    const int32_t blk = __builtin_nontemporal_load(L.bt + (int64_t)seq * L.bt_stride + (pos >> L.bs_log2));
    return ((int64_t)blk << L.bs_log2) | (int64_t)(pos & ((1 << L.bs_log2) - 1));
  }
  return (int64_t)seq * L.seq_stride + pos;
}

// ---- wave / workgroup scans ---------------------------------------------------------------
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int o = __shfl_up(v, off, 64);
    if (lane >= off) v += o;
  }
  return v;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Exclusive scan of one int per thread over a workgroup of NT threads (NT % 64 == 0).
// `tmp` needs NT/64 + 1 ints of LDS.  Returns the exclusive prefix; *total gets the sum.
template <int NT>
__device__ __forceinline__ int wg_exclusive_scan(int v, int* tmp, int* total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_inclusive_scan(v);
  if (lane == 63) tmp[wave] = incl;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int c = tmp[w];
    base += (w < wave) ? c : 0;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return base + incl - v;
}

}  // namespace dsa
