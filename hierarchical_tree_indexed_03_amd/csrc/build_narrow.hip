// Tree build for narrow reference sets (R <= 4) and small power-of-two blocks (b <= 8).
//
// Same quantities as the leaf kernel of build.hip (news summary "Zyphra releases the ZHA
// sparse attention method", section "Building the tree": per block and reference query the
// logsumexp LSE_j of the logits r_j.k / sqrt(d), the softmax-weighted mean key s_j and
// c_j = LSE_j - r_j.s_j / sqrt(d); the parent level from its children, blog "Zyphra
// Hierarchical Attention", section "Building the tree"), organised for few planes: with
// R <= 4 a contraction tile would leave most MFMA columns idle and the per-level passes of
// the leaf kernel run on a handful of threads.  Here each block of b tokens belongs to d/8
// consecutive lanes, lane c holding the block's b keys restricted to columns 8c..8c+7 in
// registers.  The logits are partial dot products reduced across those lanes; every lane
// then has the block's logits, so LSE, weights, A_j and its 8 columns of s_j follow in
// registers with no barrier.  The level-2 nodes inside the tile (b blocks each) are formed
// from the blocks' (LSE, A, s) through LDS; levels above come from the parent kernel.  The
// next tile's keys are loaded while the current one is summarised.
#include "common.hpp"
#include "kernels.hpp"
#include "route_util.hpp"

namespace zha {

namespace {

// 8 consecutive elements as floats from one (bf16) or two (fp32) 16-byte pieces
template <typename TIn> struct Row8;
template <> struct Row8<bf16_t> {
  static constexpr int NU = 1;
  __device__ static void to_f32(const uint4* u, float* o) {
    const uint32_t w[4] = {u[0].x, u[0].y, u[0].z, u[0].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) { o[2 * i] = bf16_bits_to_f32(w[i] & 0xffffu); o[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16); }
  }
};
template <> struct Row8<float> {
  static constexpr int NU = 2;
  __device__ static void to_f32(const uint4* u, float* o) {
    o[0] = __uint_as_float(u[0].x); o[1] = __uint_as_float(u[0].y); o[2] = __uint_as_float(u[0].z); o[3] = __uint_as_float(u[0].w);
    o[4] = __uint_as_float(u[1].x); o[5] = __uint_as_float(u[1].y); o[6] = __uint_as_float(u[1].z); o[7] = __uint_as_float(u[1].w);
  }
};

// MX FP4 of 8 consecutive elements per lane, a 32-element block in 4 consecutive lanes
// (lane c holds elements 8c..8c+7 of the row, all 4 lanes active): amax over the block,
// then one 32-bit word of codes per lane and the block's scale byte from its first lane.
__device__ __forceinline__ void store_fp4_x8(uint8_t* q, uint8_t* x, int64_t e, const float* v) {
  float am = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(v[i]));
  am = fmaxf(am, __shfl_xor(am, 1));
  am = fmaxf(am, __shfl_xor(am, 2));
  const uint32_t sb = mx_scale_byte(am);
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) w |= e2m1_code(v[i], sb) << (4 * i);
  *(uint32_t*)(q + e / 2) = w;
  if ((e & 31) == 0) x[e / 32] = (uint8_t)sb;
}

__device__ __forceinline__ void store_bf16x8(bf16_t* p, const float* v) {
  uint4 w;
  w.x = f2bf16_bits(v[0]) | (f2bf16_bits(v[1]) << 16);
  w.y = f2bf16_bits(v[2]) | (f2bf16_bits(v[3]) << 16);
  w.z = f2bf16_bits(v[4]) | (f2bf16_bits(v[5]) << 16);
  w.w = f2bf16_bits(v[6]) | (f2bf16_bits(v[7]) << 16);
  *(uint4*)p = w;
}

}  // namespace

template <typename TIn, int D, int R, int B>
__global__ __launch_bounds__(256) void build_narrow_kernel(BuildArgs a) {
  constexpr int CG = D / 8;                 // lanes per block (8 columns each)
  constexpr int NB = 256 / CG;              // blocks per tile
  constexpr int T = NB * B;                 // tokens per tile
  constexpr int NP = NB / B;                // level-2 nodes per tile
  constexpr int NU = Row8<TIn>::NU;         // 16-byte pieces per row slice
  constexpr int CH = 16 / sizeof(TIn);      // elements per piece
  __shared__ float Lb[NB][R], Ab[NB][R];
  __shared__ __align__(16) float Sb[NB][R][D];

  const int kv = blockIdx.y;
  // a new tree: the append's cached sibling aggregates no longer hold
  if (blockIdx.x == 0 && threadIdx.x <= MAXL) a.dev.sibkey[(int64_t)kv * (MAXL + 1) + threadIdx.x] = -1;
  const int tid = threadIdx.x, blk = tid / CG, cg = tid % CG;
  const TIn* Kg = (const TIn*)a.K + (int64_t)kv * a.cap * D;
  const TIn* Rg = (const TIn*)a.refs + (int64_t)kv * R * D;
  const int64_t N = a.N;
  const int64_t ntiles = (N + T - 1) / T;

  // sigma * r_j restricted to the lane's 8 columns
  float rq[R][8];
#pragma unroll
  for (int j = 0; j < R; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) rq[j][i] = a.sigma * to_f32(Rg[j * D + cg * 8 + i]);

  // the lane's B key rows (8 columns each) of tile `tile`, zeros past N
  uint4 kr[B][NU];
  auto load_keys = [&](int64_t tile) {
    const int64_t tb = tile * T + (int64_t)blk * B;
#pragma unroll
    for (int r = 0; r < B; ++r)
#pragma unroll
      for (int u = 0; u < NU; ++u)
        kr[r][u] = tb + r < N ? *(const uint4*)(Kg + (tb + r) * D + cg * 8 + u * CH) : make_uint4(0, 0, 0, 0);
  };
  if (a.tile0 + (int64_t)blockIdx.x < ntiles) load_keys(a.tile0 + blockIdx.x);
  for (int64_t tile = a.tile0 + blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int64_t t0 = tile * T;
    const int64_t tb = t0 + (int64_t)blk * B;   // first token of the lane's block
    float k[B][8];
#pragma unroll
    for (int r = 0; r < B; ++r) Row8<TIn>::to_f32(kr[r], k[r]);
    if (tile + gridDim.x < ntiles) load_keys(tile + gridDim.x);

    // ---- level 1: logits, LSE, weights, A and the lane's 8 columns of s, per plane
    float z[R][B];
#pragma unroll
    for (int j = 0; j < R; ++j)
#pragma unroll
      for (int r = 0; r < B; ++r) {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc += rq[j][i] * k[r][i];
        z[j][r] = acc;
      }
#pragma unroll
    for (int off = 1; off < CG; off <<= 1)
#pragma unroll
      for (int j = 0; j < R; ++j)
#pragma unroll
        for (int r = 0; r < B; ++r) z[j][r] += __shfl_xor(z[j][r], off);
    const bool exists = tb < N;
    const int nrow = exists ? (int)min((int64_t)B, N - tb) : 0;
    const int64_t n1 = tb / B;                   // level-1 node of the lane's block
    const int64_t g1 = (int64_t)kv * a.dev.ncap[1] + n1;
#pragma unroll
    for (int j = 0; j < R; ++j) {
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < B; ++r) if (r < nrow) mx = fmaxf(mx, z[j][r]);
      float sum = 0.f;
#pragma unroll
      for (int r = 0; r < B; ++r) if (r < nrow) sum += expf(z[j][r] - mx);
      const float lse = exists ? mx + logf(sum) : -INFINITY;
      float w[B], A = 0.f, s[8];
#pragma unroll
      for (int r = 0; r < B; ++r) {
        w[r] = r < nrow ? expf(z[j][r] - lse) : 0.f;
        A += w[r] * (r < nrow ? z[j][r] : 0.f);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float acc = 0.f;
#pragma unroll
        for (int r = 0; r < B; ++r) acc += w[r] * k[r][i];
        s[i] = acc;
      }
      if (exists) {
        const int64_t so = (g1 * R + j) * D + cg * 8;
        *(float4*)(a.dev.s[1] + so) = make_float4(s[0], s[1], s[2], s[3]);
        *(float4*)(a.dev.s[1] + so + 4) = make_float4(s[4], s[5], s[6], s[7]);
        if (a.dev.sq[1]) store_bf16x8(a.dev.sq[1] + so, s);
        if (cg == 0) {
          a.dev.c[1][g1 * R + j] = lse - A;
          a.dev.lse[1][g1 * R + j] = lse;
        }
        if (a.dev.w1 && cg == 0)
#pragma unroll
          for (int r = 0; r < B; ++r) a.dev.w1[(g1 * R + j) * B + r] = w[r];
      }
      // FP4 copy (a 4-lane MX group lies within one block, whose lanes share `exists`)
      if (a.dev.s4[1] && exists) store_fp4_x8(a.dev.s4[1], a.dev.s4x[1], (g1 * R + j) * D + cg * 8, s);
      if (cg == 0) {
        Lb[blk][j] = lse;
        Ab[blk][j] = A;
      }
#pragma unroll
      for (int i = 0; i < 8; i += 4) *(float4*)&Sb[blk][j][cg * 8 + i] = make_float4(s[i], s[i + 1], s[i + 2], s[i + 3]);
    }
    __syncthreads();

    // ---- level 2 inside the tile: node p from blocks p*B .. p*B+B-1
    if (a.m >= 2) {
      for (int idx = tid; idx < NP * R * (D / 4); idx += 256) {
        const int p = idx / (R * (D / 4)), j = (idx / (D / 4)) % R, dc = idx % (D / 4);
        const int64_t first_tok = t0 + (int64_t)p * B * B;
        float mx = -INFINITY;
#pragma unroll
        for (int c = 0; c < B; ++c) mx = fmaxf(mx, Lb[p * B + c][j]);
        const bool ex2 = first_tok < N;
        float sum = 0.f;
        if (ex2)
#pragma unroll
          for (int c = 0; c < B; ++c) sum += expf(Lb[p * B + c][j] - mx);
        const float lse2 = ex2 ? mx + logf(sum) : -INFINITY;
        float A2 = 0.f;
        float4 s2 = make_float4(0.f, 0.f, 0.f, 0.f);
        if (ex2)
#pragma unroll
          for (int c = 0; c < B; ++c) {
            const float e = expf(Lb[p * B + c][j] - lse2);
            A2 += e * Ab[p * B + c][j];
            const float4 v = *(const float4*)&Sb[p * B + c][j][dc * 4];
            s2.x += e * v.x; s2.y += e * v.y; s2.z += e * v.z; s2.w += e * v.w;
          }
        const int64_t n2 = first_tok / (B * B);
        const int64_t g2 = (int64_t)kv * a.dev.ncap[2] + n2;
        const int64_t so = (g2 * R + j) * D + dc * 4;
        if (ex2) {
          *(float4*)(a.dev.s[2] + so) = s2;
          if (a.dev.sq[2]) {
            uint2 w;
            w.x = f2bf16_bits(s2.x) | (f2bf16_bits(s2.y) << 16);
            w.y = f2bf16_bits(s2.z) | (f2bf16_bits(s2.w) << 16);
            *(uint2*)(a.dev.sq[2] + so) = w;
          }
          if (dc == 0) {
            a.dev.c[2][g2 * R + j] = lse2 - A2;
            a.dev.lse[2][g2 * R + j] = lse2;
          }
        }
        if (a.dev.s4[2]) {
          // 8 consecutive lanes hold one 32-element MX block (items run dc fastest)
          float am = fmaxf(fmaxf(fabsf(s2.x), fabsf(s2.y)), fmaxf(fabsf(s2.z), fabsf(s2.w)));
          am = fmaxf(am, __shfl_xor(am, 1));
          am = fmaxf(am, __shfl_xor(am, 2));
          am = fmaxf(am, __shfl_xor(am, 4));
          const uint32_t sb = mx_scale_byte(am);
          const uint32_t cw = e2m1_code(s2.x, sb) | (e2m1_code(s2.y, sb) << 4) | (e2m1_code(s2.z, sb) << 8) |
                              (e2m1_code(s2.w, sb) << 12);
          if (ex2) {
            *(uint16_t*)(a.dev.s4[2] + so / 2) = (uint16_t)cw;
            if ((dc & 7) == 0) a.dev.s4x[2][so / 32] = (uint8_t)sb;
          }
        }
      }
    }
    __syncthreads();
  }
}

// Host side: grids of one wave of resident workgroups, persistent over the tiles.
template <typename TIn, int D, int R, int B>
static void launch_narrow_t(const BuildArgs& a, int hkv, hipStream_t st) {
  constexpr int T = (256 / (D / 8)) * B;
  static const int per_cu = resident_per_cu(build_narrow_kernel<TIn, D, R, B>, 256);
  const int64_t ntiles = (a.N + T - 1) / T;
  int64_t x = (int64_t)per_cu * device_cus() / hkv;
  if (x > ntiles - a.tile0) x = ntiles - a.tile0;
  if (x < 1) x = 1;
  hipLaunchKernelGGL((build_narrow_kernel<TIn, D, R, B>), dim3((unsigned)x, (unsigned)hkv), dim3(256), 0, st, a);
}

bool narrow_build(int R, int b) { return R <= 4 && (b == 2 || b == 4 || b == 8); }

int narrow_tile_tokens(int D, int b) { return (256 / (D / 8)) * b; }

template <typename TIn, int D>
static hipError_t launch_narrow_d(const BuildArgs& a, int R, int hkv, hipStream_t st) {
#define ZHA_CASE(RR, BB) if (R == RR && a.b == BB) { launch_narrow_t<TIn, D, RR, BB>(a, hkv, st); return hipGetLastError(); }
  ZHA_CASE(1, 2) ZHA_CASE(1, 4) ZHA_CASE(1, 8)
  ZHA_CASE(2, 2) ZHA_CASE(2, 4) ZHA_CASE(2, 8)
  ZHA_CASE(4, 2) ZHA_CASE(4, 4) ZHA_CASE(4, 8)
#undef ZHA_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_build_narrow(const BuildArgs& a, bool bf16, int D, int R, int hkv, hipStream_t st) {
  if (bf16) return D == 64 ? launch_narrow_d<bf16_t, 64>(a, R, hkv, st) : launch_narrow_d<bf16_t, 128>(a, R, hkv, st);
  return D == 64 ? launch_narrow_d<float, 64>(a, R, hkv, st) : launch_narrow_d<float, 128>(a, R, hkv, st);
}

}  // namespace zha
