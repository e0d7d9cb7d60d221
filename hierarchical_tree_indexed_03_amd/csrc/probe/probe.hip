// Measurement kernels for the benchmark (not part of the ZHA path): a streaming read of a
// device buffer (the practical HBM read ceiling on this GPU) and a plain copy of known size
// (used to scale hardware traffic counters to bytes).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ p, int64_t n, uint32_t* out) {
  uint32_t acc = 0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 7 * stride < n; i += 8 * stride) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p[i + u * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n; i += stride) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9e3779b9u) out[blockIdx.x] = acc;   // practically never taken; keeps the loads live
}

__global__ __launch_bounds__(256) void copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16) from `p`; `sink` needs 4 * blocks bytes.  Returns a
// hipError_t code.
int zha_probe_stream_read(const void* p, int64_t bytes, void* sink, int blocks, hipStream_t st) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, st, (const uint4*)p, bytes / 16, (uint32_t*)sink);
  return (int)hipGetLastError();
}

// Copies `bytes` (a multiple of 16) from src to dst.
int zha_probe_copy(const void* src, void* dst, int64_t bytes, int blocks, hipStream_t st) {
  hipLaunchKernelGGL(copy_kernel, dim3(blocks), dim3(256), 0, st, (const uint4*)src, (uint4*)dst, bytes / 16);
  return (int)hipGetLastError();
}

}
