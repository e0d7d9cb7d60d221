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

// Row swaps (gfx950): permlane16_swap exchanges the odd 16-lane rows of x with the even rows
// of y; permlane32_swap exchanges the upper 32 lanes of x with the lower 32 lanes of y.
__device__ __forceinline__ void swap_rows16(float& x, float& y) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  x = __uint_as_float(r[0]);
  y = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap_rows32(float& x, float& y) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  x = __uint_as_float(r[0]);
  y = __uint_as_float(r[1]);
}

// Maxima over the 4 lane rows of NP per-lane values m[0..NP) (one per node).  On return
// row r holds in out[i], i < max(NP/4, 1), the maximum of node key_row_node<NP>(i, r).
//   step 1 (rows r, r^1): pairs (m[i], m[i + NP/2]); a row of parity p keeps node i + p*NP/2
//   step 2 (rows r, r^2): pairs (A[i], A[i + NA/2]); rows 0, 1 keep the first, rows 2, 3 the
//   second, each for its parity
template <int NP>
__device__ __forceinline__ int key_row_node(int i, int r) {
  constexpr int NA = NP >= 2 ? NP / 2 : 1;
  const int j = NA >= 2 ? i + (r >= 2 ? NA / 2 : 0) : i;
  return NP >= 2 ? j + (r & 1) * (NP / 2) : 0;
}
template <int NP>
__device__ __forceinline__ void key_row_max(const float (&m)[NP], float (&out)[NP >= 4 ? NP / 4 : 1]) {
  constexpr int NA = NP >= 2 ? NP / 2 : 1;
  float A[NA];
  if constexpr (NP >= 2) {
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      float x = m[i], y = m[i + NA];
      swap_rows16(x, y);
      A[i] = fmaxf(x, y);
    }
  } else {
    float x = m[0], y = m[0];
    swap_rows16(x, y);
    A[0] = fmaxf(x, y);
  }
  if constexpr (NA >= 2) {
#pragma unroll
    for (int i = 0; i < NA / 2; ++i) {
      float x = A[i], y = A[i + NA / 2];
      swap_rows32(x, y);
      out[i] = fmaxf(x, y);
    }
  } else {
    float x = A[0], y = A[0];
    swap_rows32(x, y);
    out[0] = fmaxf(x, y);
  }
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
