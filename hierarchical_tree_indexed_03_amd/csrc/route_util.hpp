// Device helpers shared by the router kernels.
#pragma once
#include "common.hpp"

namespace zha {

// Orders the LDS traffic of one wave (a wave-wide barrier with release/acquire fences).
__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Rank order of the top-p selection as one integer: higher score first, equal scores by
// lower node position (ascending key = rank order).
__device__ __forceinline__ uint64_t rank_key(float s, int32_t e) {
  return ((uint64_t)(~f2key(s)) << 32) | (uint32_t)e;
}

// Compute units of the current device (queried once per process).
static inline int device_cus() {
  static const int ncu = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 256;
    return n > 0 ? n : 256;
  }();
  return ncu;
}

// Workgroups of a kernel resident on one compute unit at once (queried once per kernel).
template <typename F>
static inline int resident_per_cu(F kernel, int threads) {
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, threads, 0) != hipSuccess || nb < 1) nb = 1;
  return nb;
}

static inline unsigned grid_for(int64_t n, int64_t per, int64_t cap) {
  int64_t x = (n + per - 1) / per;
  if (x > cap) x = cap;
  return (unsigned)(x < 1 ? 1 : x);
}

}  // namespace zha
