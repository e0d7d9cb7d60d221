// K.Q^T tiles on MFMA, shared by the attention kernel and the key-form level-1 scoring.
#pragma once
#include "common.hpp"

namespace zha {

// S^T tile = K (16 tokens x D) . Q^T (D x 16 heads) on MFMA; the contraction index is
// permuted so each lane reads one contiguous D/4 slice of its token's key row.
template <typename TIn, int D> struct Qk;
template <int D> struct Qk<bf16_t, D> {
  static constexpr int NL = D / 32;           // 16-byte loads per lane per 16-token tile
  bf16x8 q[NL];
  __device__ void load_q(const bf16_t* qg, int g, int col, int kg) {
#pragma unroll
    for (int kk = 0; kk < NL; ++kk) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (col < g) v = *(const uint4*)(qg + col * D + kg * (D / 4) + kk * 8);
      q[kk] = __builtin_bit_cast(bf16x8, v);
    }
  }
  __device__ static void load_k(const bf16_t* krow, int kg, uint4* k) {
#pragma unroll
    for (int kk = 0; kk < NL; ++kk) k[kk] = *(const uint4*)(krow + kg * (D / 4) + kk * 8);
  }
  __device__ f32x4 mma(const uint4* k) const {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < NL; ++kk)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k[kk]), q[kk], acc, 0, 0, 0);
    return acc;
  }
};
template <int D> struct Qk<float, D> {
  static constexpr int NL = D / 16;           // float4 loads per lane per tile
  float q[D / 4];
  __device__ void load_q(const float* qg, int g, int col, int kg) {
#pragma unroll
    for (int i = 0; i < D / 4; ++i) q[i] = col < g ? qg[col * D + kg * (D / 4) + i] : 0.f;
  }
  __device__ static void load_k(const float* krow, int kg, uint4* k) {
#pragma unroll
    for (int i = 0; i < NL; ++i) k[i] = *(const uint4*)(krow + kg * (D / 4) + i * 4);
  }
  __device__ f32x4 mma(const uint4* k) const {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(k[i].x), q[4 * i + 0], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(k[i].y), q[4 * i + 1], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(k[i].z), q[4 * i + 2], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(k[i].w), q[4 * i + 3], acc, 0, 0, 0);
    }
    return acc;
  }
};

}  // namespace zha
