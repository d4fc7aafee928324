// dsa_indexer_topk_noalloc: the indexer + Top-K call with its workspace in a file-scope device
// array instead of a caller buffer, for callers that cannot allocate device memory.
//
// `scratch` is one array per device (each device that loads this library holds its own copy,
// at its own address, until the process ends).  In host code its name is only a stand-in for
// the device symbol, so the host never passes it to a kernel or a copy: at a device's first
// call, with that device current, hipGetSymbolAddress gives the array's device address, which
// is kept per device and used from then on.  That first call also enqueues a fill kernel that
// zeroes the array on the caller's stream (the indexer's arrival counters must start at zero;
// every call leaves them zero again), so it is ordered before the indexer that follows.
// Every call on one device shares the array: calls that overlap on one device race.

#include <mutex>

#include "../../include/dsa.h"
#include "dsa_internal.hpp"

namespace dsa {
namespace {

static_assert(DSA_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) uint8_t scratch[DSA_NOALLOC_SCRATCH_BYTES];

__global__ __launch_bounds__(256) void scratch_clear_kernel(uint4* p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
    p[i] = uint4{0u, 0u, 0u, 0u};
}

std::mutex g_mutex;
void* g_ptr[kMaxDevices] = {};

// The device address of this device's scratch array; the first call on a device also
// enqueues its clearing on `stream`.
hipError_t scratch_of_current_device(hipStream_t stream, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    hipLaunchKernelGGL(scratch_clear_kernel, dim3(1024), dim3(256), 0, stream,
                       static_cast<uint4*>(ptr), (size_t)DSA_NOALLOC_SCRATCH_BYTES / 16);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    g_ptr[dev] = ptr;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace
}  // namespace dsa

extern "C" dsa_status dsa_indexer_topk_noalloc(
    const void* q, dsa_dtype q_dtype, const float* head_w, const void* k_pool, dsa_dtype k_dtype,
    const float* k_scale, int32_t n_heads, int32_t head_dim, const dsa_layout* layout,
    const dsa_queries* queries, int32_t top_k, int32_t* out_idx, float* out_score,
    void* stream) {
  // the same argument checks as the workspace entry point, before anything touches a device
  const dsa_status pre = dsa_indexer_topk(q, q_dtype, head_w, k_pool, k_dtype, k_scale, n_heads,
                                          head_dim, layout, queries, top_k, out_idx, out_score,
                                          nullptr, 0, nullptr);
  if (pre != DSA_ERR_WORKSPACE) return pre;   // any other status: an argument error
  const dsa::IndexerPlan pl =
      dsa::plan_indexer(queries->num_queries, queries->max_visible, top_k, queries->total_visible);
  if (pl.bytes > (size_t)DSA_NOALLOC_SCRATCH_BYTES) return DSA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (dsa::scratch_of_current_device(static_cast<hipStream_t>(stream), &ws) != hipSuccess)
    return DSA_ERR_HIP;
  return dsa_indexer_topk(q, q_dtype, head_w, k_pool, k_dtype, k_scale, n_heads, head_dim, layout,
                          queries, top_k, out_idx, out_score, ws, DSA_NOALLOC_SCRATCH_BYTES, stream);
}
