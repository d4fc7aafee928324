// Indexer prolog: the indexer's query, key and head weights from a token's hidden vector,
// the key's RMSNorm, the query's quantization and the key's cache store ("Day0 Adaptation and
// Performance Optimization for Novel Long-Sequence Reasoning Models", section 3; "Large Model
// Inference Acceleration: Day-0 Adaptation...", section 1.2; "Optimizing and Deploying
// Ultra-Long Sequence Inference Architectures", section I).
//
// The pages run the projections and the normalization on parallel streams so that the small
// steps overlap.  Here the three projections read the same hidden vector, so they are one
// GEMM over a weight matrix whose columns are the query (head-major), the key and the head
// weights: one pass over x and W, one library GEMM (bf16 in, fp32 out), and one epilogue
// kernel that rounds or MXFP8-quantizes the query (2048 values a workgroup), copies the head
// weights, RMS-normalizes the key and writes it into the paged key pool in its storage format.
#include <mutex>

#include <rocblas/rocblas.h>

#include "store_row.hpp"

namespace dsa {
namespace {

constexpr int kPrologThreads = 256;
constexpr int kQPerBlock = kPrologThreads * 8;   // query values of one workgroup

// Grid (T, QB + 1): blocks y < QB take 2048 query values of token x (8 per thread, loads
// issued together and coalesced); block QB takes the head weights and the key.
__global__ __launch_bounds__(kPrologThreads) void prolog_epilogue_kernel(PrologParams p) {
  __shared__ float kr[kPrologMaxD];
  __shared__ float red[kPrologThreads / 64];
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* y = p.y + (size_t)t * p.N;
  const int HD = p.H * p.D;
  if ((int)blockIdx.y < (int)gridDim.y - 1) {
    // value e of this thread: index blockIdx.y * 2048 + 256 e + tid (each load and store
    // instruction covers consecutive values)
    const int i0 = (int)blockIdx.y * kQPerBlock + tid;
    uint16_t* q = (uint16_t*)p.q_out + (size_t)t * HD;
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = i0 + 256 * e < HD ? y[i0 + 256 * e] : 0.f;
    if (p.q_mx) {
      // MXFP8 per head and group of 32 dims: 32 lanes hold a group for each e (HD % 32 == 0,
      // so a group never straddles the end); the dequantized value code * 2^(byte - 127) is
      // exact in bf16 for scale bytes >= 3
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float amax = fabsf(v[e]);
#pragma unroll
        for (int off = 16; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
        const uint32_t sb = mx_scale_byte(amax);
        v[e] = fp8_e4m3_to_f32(f32_to_fp8_e4m3(v[e] * mx_inv_scale(sb))) * mx_scale_f32(sb);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (i0 + 256 * e < HD) q[i0 + 256 * e] = (uint16_t)f32_to_bf16_bits(v[e]);
    return;
  }
  for (int i = tid; i < p.H; i += kPrologThreads) p.w_out[(size_t)t * p.H + i] = y[HD + p.D + i];
  // key: k / sqrt(mean(k^2) + eps) * gain
  float ss = 0.f;
  for (int i = tid; i < p.D; i += kPrologThreads) {
    const float v = y[HD + i];
    kr[i] = v;
    ss += v * v;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < kPrologThreads / 64; ++w) tot += red[w];
  const float r = 1.0f / sqrtf(tot / (float)p.D + p.eps);
  for (int i = tid; i < p.D; i += kPrologThreads) {
    const float k = kr[i] * r * p.gain[i];
    kr[i] = k;
    if (p.k_out) p.k_out[(size_t)t * p.D + i] = k;
  }
  __syncthreads();
  if (p.pool && wave == 0) store_key_row(kr, p.D, p.slot[t], p.pool, p.k_dt, p.k_scale, lane);
}

std::mutex g_blas_mutex;
rocblas_handle g_blas[kMaxDevices] = {};

}  // namespace

// Y[T, N] = x[T, d_x] W[d_x, N], all row-major: in rocBLAS's column-major terms Y^T = W^T x^T
// with W^T an N x d_x matrix of leading dimension N and x^T a d_x x T one of leading
// dimension d_x.
hipError_t run_prolog(const void* x, int32_t T, int32_t d_x, const void* w_proj,
                      const PrologParams& p, hipStream_t stream, int* blas_status) {
  *blas_status = 0;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  {
    std::lock_guard<std::mutex> lock(g_blas_mutex);
    if (!g_blas[dev]) {
      const rocblas_status s = rocblas_create_handle(&g_blas[dev]);
      if (s != rocblas_status_success) {
        g_blas[dev] = nullptr;
        *blas_status = (int)s;
        return hipSuccess;
      }
    }
    rocblas_handle h = g_blas[dev];
    rocblas_status s = rocblas_set_stream(h, stream);
    const float alpha = 1.f, beta = 0.f;
    if (s == rocblas_status_success)
      s = rocblas_gemm_ex(h, rocblas_operation_none, rocblas_operation_none, p.N, T, d_x, &alpha,
                          w_proj, rocblas_datatype_bf16_r, p.N, x, rocblas_datatype_bf16_r, d_x,
                          &beta, (void*)p.y, rocblas_datatype_f32_r, p.N, (void*)p.y,
                          rocblas_datatype_f32_r, p.N, rocblas_datatype_f32_r,
                          rocblas_gemm_algo_standard, 0, 0);
    if (s != rocblas_status_success) {
      *blas_status = (int)s;
      return hipSuccess;
    }
  }
  const int qb = (p.H * p.D + kQPerBlock - 1) / kQPerBlock;
  hipLaunchKernelGGL(prolog_epilogue_kernel, dim3(T, qb + 1), dim3(kPrologThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace dsa
