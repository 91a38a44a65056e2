// Streaming read and copy kernels used to measure the achievable HBM rate and to calibrate byte counters.
#include <stdint.h>

#include "../../include/pa.h"
#include "../../include/paged_attention_diag.h"
#include "pa_device.h"

namespace pa {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;  // 16-byte loads in flight per lane per iteration

// Workgroups take contiguous chunks of kThreads * kUnroll words; each lane's kUnroll loads are issued
// before any is used. The xor of everything a lane read is folded per workgroup and stored in sink so that
// no load can be dropped.
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const U4* __restrict__ src, int64_t words,
                                                               float* __restrict__ sink) {
  uint32_t x = 0;
  const int64_t step = (int64_t)gridDim.x * kThreads * kUnroll;
  for (int64_t base = (int64_t)blockIdx.x * kThreads * kUnroll; base < words; base += step) {
    U4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + u * kThreads + threadIdx.x;
      v[u] = i < words ? load_stream(reinterpret_cast<const char*>(src + i)) : U4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  __shared__ uint32_t red[kThreads / kWave];
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) x ^= __shfl_xor(x, off);
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t y = 0;
    for (int w = 0; w < kThreads / kWave; ++w) y ^= red[w];
    sink[blockIdx.x] = __uint_as_float(y);
  }
}

__global__ __launch_bounds__(kThreads) void stream_copy_kernel(U4* __restrict__ dst, const U4* __restrict__ src,
                                                               int64_t words) {
  const int64_t step = (int64_t)gridDim.x * kThreads * kUnroll;
  for (int64_t base = (int64_t)blockIdx.x * kThreads * kUnroll; base < words; base += step) {
    U4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + u * kThreads + threadIdx.x;
      if (i < words) v[u] = load_stream(reinterpret_cast<const char*>(src + i));
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + u * kThreads + threadIdx.x;
      if (i < words) dst[i] = v[u];
    }
  }
}

unsigned grid_for(int64_t words) {
  const int64_t per_wg = (int64_t)kThreads * kUnroll;
  const int64_t need = (words + per_wg - 1) / per_wg;
  return (unsigned)(need < PA_STREAM_SINK_FLOATS ? need : PA_STREAM_SINK_FLOATS);
}

}  // namespace
}  // namespace pa

extern "C" {

int pa_stream_read(const void* src, size_t bytes, float* sink, void* stream) {
  if (bytes == 0 || bytes % 16 != 0) return PA_ERR_SHAPE;
  if (!src || !sink) return PA_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(src) & 15u) || (reinterpret_cast<uintptr_t>(sink) & 3u)) return PA_ERR_ALIGN;
  const int64_t words = (int64_t)(bytes / 16);
  pa::stream_read_kernel<<<pa::grid_for(words), pa::kThreads, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const pa::U4*>(src), words, sink);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int pa_stream_copy(void* dst, const void* src, size_t bytes, void* stream) {
  if (bytes == 0 || bytes % 16 != 0) return PA_ERR_SHAPE;
  if (!src || !dst) return PA_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(src) & 15u) || (reinterpret_cast<uintptr_t>(dst) & 15u)) return PA_ERR_ALIGN;
  const int64_t words = (int64_t)(bytes / 16);
  pa::stream_copy_kernel<<<pa::grid_for(words), pa::kThreads, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<pa::U4*>(dst), static_cast<const pa::U4*>(src), words);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // extern "C"
