// Router scores of every level from the keys, for deep trees (block 4, many reference
// queries): one pass over the key cache instead of the planes of every level.
//
// A node's router score is max_j (q.s_j / sqrt(d) + c_j) over its reference planes (news
// summary "Zyphra releases the ZHA sparse attention method", section "Building the tree";
// blog "Zyphra Hierarchical Attention", section "Routing through the tree").  The tree keeps
// per node and plane the log mass LSE_j at r_j besides s_j and c_j.  A parent's s_j is its
// children's s_j weighted by exp(LSE_cj - LSE_j), and a level-1 node's s_j its keys weighted
// by the token weights w_jt = exp(r_j.k_t / sqrt(d) - LSE_j).  With
// D_j(q) = q.s_j / sqrt(d) the dot products therefore follow from the keys upwards:
//   level 1:  D_j = sum_t w_jt (q.k_t / sqrt(d))
//   level l:  D_j = sum_c exp(LSE_cj - LSE_j) D_cj
// and every level's scores come from one pass over the group's logits q.k_t and the
// per-node (c, LSE) vectors.  For block 4 and R planes of d-vectors the pass reads
// d*2 + R*4 bytes per token plus 8R per node, against R*(d+1)*4 per node for the planes of
// every level (a level-1 plane alone covers 4 tokens).
//
// GPU organisation.  A workgroup takes one level-4 node (256 tokens) of one KV head and its
// four waves one level-3 node (64 tokens) each.  A wave issues every load of its 64 tokens
// at once: the keys (each lane a contiguous quarter of one key row), the level-1 token
// weights in the MFMA operand layout, and the (c, LSE) vectors of its level-1..3 nodes as
// coalesced 16-byte pieces staged through LDS.  Per 16-token tile: S^T = K.Q^T on bf16 MFMA
// (tokens x heads), a 4x4 transpose across lane rows on the gfx950 row swaps, then one fp32
// MFMA per level-1 node, [planes x tokens] . [tokens x heads], so a lane holds 4 planes of
// one head of every node.  The levels above combine in registers; level 4 combines the four
// waves' level-3 dot products through LDS.  Its dot products (per head and plane) go to
// dev.kdots, from which the top-down selection derives the levels above.
#include "common.hpp"
#include "kernels.hpp"
#include "route_util.hpp"
#include "qk_tile.hpp"

namespace zha {

// 4x4 transpose of (lane row, element): on return v[i] in row r is the old v[r] of row i.
__device__ __forceinline__ void rows_transpose4(float (&v)[4]) {
  swap_rows16(v[0], v[1]);
  swap_rows16(v[2], v[3]);
  swap_rows32(v[0], v[2]);
  swap_rows32(v[1], v[3]);
}

__device__ __forceinline__ f32x4 lds4(const float* p) { return *(const f32x4*)p; }

template <int D, int R>
__global__ __launch_bounds__(256, 4) void route_score_allkeys_kernel(RouteArgs a) {
  static_assert(R % 4 == 0 && R <= 16, "planes in whole lane rows");
  constexpr int B = AK_B;
  constexpr int NK = Qk<bf16_t, D>::NL;
  constexpr int NV = R / 4;                 // lane rows holding planes 4kg..4kg+3
  // per wave: c and LSE of its 16 level-1 nodes, 4 level-2 nodes and its level-3 node
  constexpr int S1 = 16 * R, S2 = 4 * R, S3 = R;
  constexpr int SW = 2 * (S1 + S2 + S3);    // floats staged per wave
  __shared__ __align__(16) float P[4][SW];
  __shared__ __align__(16) f32x4 W4[4][64];
  const int kv = blockIdx.y, u = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, kg = lane >> 4;
  const int g = a.g;
  const int64_t N = a.N;
  const int64_t n1l = a.nl[1], n2l = a.nl[2], n3l = a.nl[3];
  const int64_t cap1 = a.dev.ncap[1], cap2 = a.dev.ncap[2], cap3 = a.dev.ncap[3], cap4 = a.dev.ncap[4];
  const int64_t n3 = (int64_t)u * 4 + wave;     // this wave's level-3 node
  const int64_t n2b = n3 * 4, n1b = n3 * 16;    // its first level-2 and level-1 nodes
  const float sigma = a.sigma;
  const bool rowv = kg < NV;                     // this lane row holds real planes
  const int pr = 4 * (rowv ? kg : NV - 1);       // first plane of the lane row (clamped)

  // the route prep of this path: every level's list size (the whole level; level 0, the
  // gather list, is written by the selection) and the selection's arrival counts cleared
  if (a.prep_fold && u == 0 && kv == 0) {
    for (int i = threadIdx.x; i < (MAXL + 1) * a.hkv; i += blockDim.x) {
      const int lv = i / a.hkv;
      const int32_t n = (lv >= 1 && lv <= a.levels) ? (int32_t)a.nl[lv] : 0;
      a.dev.cnt[i] = n;
      a.dev.ucnt[i] = n;
    }
    for (int i = threadIdx.x; i < a.hkv; i += blockDim.x) a.dev.tick[i] = 0u;
  }

  Qk<bf16_t, D> qk;
  qk.load_q((const bf16_t*)a.q + (int64_t)kv * g * D, g, col, kg);

  // ---- every load of the wave's 64 tokens, issued before any is used
  // (c, LSE) vectors: 16-byte pieces, staged [c1 | lse1 | c2 | lse2 | c3 | lse3]
  constexpr int NP = SW / 4;                     // pieces per wave
  constexpr int NPL = (NP + 63) / 64;            // pieces per lane
  const float* sc1 = a.dev.c[1] + (kv * cap1 + n1b) * R;
  const float* sl1 = a.dev.lse[1] + (kv * cap1 + n1b) * R;
  const float* sc2 = a.dev.c[2] + (kv * cap2 + n2b) * R;
  const float* sl2 = a.dev.lse[2] + (kv * cap2 + n2b) * R;
  const float* sc3 = a.dev.c[3] + (kv * cap3 + n3) * R;
  const float* sl3 = a.dev.lse[3] + (kv * cap3 + n3) * R;
  u32x4 pv[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    int p = lane + 64 * i;
    p = p < NP ? p : NP - 1;
    // piece p of the staged layout: which array and where in it (selects, no indexed array)
    const int f = 4 * p;
    const float* src = f < S1 ? sc1 + f
                     : f < 2 * S1 ? sl1 + (f - S1)
                     : f < 2 * S1 + S2 ? sc2 + (f - 2 * S1)
                     : f < 2 * S1 + 2 * S2 ? sl2 + (f - 2 * S1 - S2)
                     : f < 2 * S1 + 2 * S2 + S3 ? sc3 + (f - 2 * S1 - 2 * S2)
                     : sl3 + (f - 2 * S1 - 2 * S2 - S3);
    pv[i] = *(const u32x4*)src;
  }
  // keys: tile s, token row col of it (rows past the cache's end read the last key; their
  // token weights are exact zeros)
  const bf16_t* Kc = (const bf16_t*)a.K + (int64_t)kv * a.kcap * D;
  uint4 kf[4][NK];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    int64_t tok = n1b * B + 16 * s + col;
    tok = tok < N ? tok : N - 1;
    Qk<bf16_t, D>::load_k(Kc + tok * D, kg, kf[s]);
  }
  // token weights, A operand of the level-1 products: lane (plane col, token kg)
  const float* W = a.dev.w1 + (kv * cap1 + n1b) * R * B;
  float wv[16];
#pragma unroll
  for (int n = 0; n < 16; ++n) wv[n] = W[(n * R + (col < R ? col : R - 1)) * B + kg];
#pragma unroll
  for (int n = 0; n < 16; ++n) wv[n] = col < R ? wv[n] : 0.f;
  // the level-4 node's c and LSE for the lane row's planes (a broadcast load)
  const f32x4 c4 = *(const f32x4*)(a.dev.c[4] + (kv * cap4 + u) * R + pr);
  const f32x4 l4 = *(const f32x4*)(a.dev.lse[4] + (kv * cap4 + u) * R + pr);

  float* Pw = P[wave];
#pragma unroll
  for (int i = 0; i < NPL; ++i)
    if (lane + 64 * i < NP) *(u32x4*)(Pw + 4 * (lane + 64 * i)) = pv[i];
  wave_sync_lds();
  const float* C1 = Pw;
  const float* L1 = Pw + S1;
  const float* C2 = Pw + 2 * S1;
  const float* L2 = Pw + 2 * S1 + S2;
  const float* C3 = Pw + 2 * S1 + 2 * S2;
  const float* L3 = Pw + 2 * S1 + 2 * S2 + S3;

  float* out1 = a.dev.score[1] + (int64_t)kv * GMAX * cap1;
  float* out2 = a.dev.score[2] + (int64_t)kv * GMAX * cap2;
  float* out3 = a.dev.score[3] + (int64_t)kv * GMAX * cap3;
  float* out4 = a.dev.score[4] + (int64_t)kv * GMAX * cap4;
  const bool hv = col < g;

  // max over the lane's valid planes of D + c
  auto pmax = [&](const f32x4& d, const f32x4& c) {
    float m = -INFINITY;
#pragma unroll
    for (int e = 0; e < 4; ++e) m = fmaxf(m, d[e] + c[e]);
    return rowv ? m : -INFINITY;
  };
  auto wsum = [&](f32x4& acc, const f32x4& d, const f32x4& lc, const f32x4& lp) {
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += expf(lc[e] - lp[e]) * d[e];
  };

  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  const f32x4 l3 = lds4(L3 + pr);
  f32x4 acc3 = zero;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int64_t n2 = n2b + s;
    const f32x4 st = qk.mma(kf[s]);             // S^T[token 4kg+e][head col]
    float v[4] = {sigma * st[0], sigma * st[1], sigma * st[2], sigma * st[3]};
    rows_transpose4(v);                         // v[i]: token 4i + kg of the tile, head col
    f32x4 d1[4];
    float m[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      d1[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(wv[4 * s + i], v[i], zero, 0, 0, 0);
      m[i] = pmax(d1[i], lds4(C1 + (4 * s + i) * R + pr));
    }
    // level-1 scores: row kg ends with node key_row_node<4>(0, kg) of the tile
    float mo[1];
    key_row_max<4>(m, mo);
    {
      const int64_t n1 = n1b + 4 * s + key_row_node<4>(0, kg);
      if (hv && n1 < n1l) out1[(int64_t)col * cap1 + n1] = mo[0];
    }
    // level 2: the tile's node
    const f32x4 l2 = lds4(L2 + s * R + pr);
    f32x4 d2 = zero;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (n1b + 4 * s + i < n1l) wsum(d2, d1[i], lds4(L1 + (4 * s + i) * R + pr), l2);
    float m2[1] = {pmax(d2, lds4(C2 + s * R + pr))}, o2[1];
    key_row_max<1>(m2, o2);
    if (hv && kg == 0 && n2 < n2l) out2[(int64_t)col * cap2 + n2] = o2[0];
    if (n2 < n2l) wsum(acc3, d2, l2, l3);
  }
  // level 3: the wave's node
  {
    float m3[1] = {pmax(acc3, lds4(C3 + pr))}, o3[1];
    key_row_max<1>(m3, o3);
    if (hv && kg == 0 && n3 < n3l) out3[(int64_t)col * cap3 + n3] = o3[0];
  }
  // level 4: the workgroup's node, from the four waves' weighted level-3 products
  f32x4 t = zero;
  if (n3 < n3l) wsum(t, acc3, l3, l4);
  W4[wave][lane] = t;
  __syncthreads();
  if (wave == 0) {
    f32x4 d4 = W4[0][lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      const f32x4 x = W4[w][lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) d4[e] += x[e];
    }
    float m4[1] = {pmax(d4, c4)}, o4[1];
    key_row_max<1>(m4, o4);
    if (hv && kg == 0) out4[(int64_t)col * cap4 + u] = o4[0];
    // the level-4 dot products, [Hkv][ncap4][GMAX][R], for the levels above
    if (hv && rowv) *(f32x4*)(a.dev.kdots + ((kv * cap4 + u) * GMAX + col) * R + 4 * kg) = d4;
  }
}

template <int D, int R>
static void launch_allkeys_t(const RouteArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((route_score_allkeys_kernel<D, R>), dim3((unsigned)a.nl[AK_LC], (unsigned)a.hkv), dim3(256), 0,
                     st, a);
}

hipError_t launch_route_allkeys_score(const RouteArgs& a, int D, int R, hipStream_t st) {
#define ZHA_CASE(DD, RR) else if (D == DD && R == RR) launch_allkeys_t<DD, RR>(a, st);
  if (false) {}
  ZHA_CASE(64, 4) ZHA_CASE(64, 8) ZHA_CASE(64, 16)
  ZHA_CASE(128, 4) ZHA_CASE(128, 8) ZHA_CASE(128, 16)
  else return hipErrorInvalidValue;
#undef ZHA_CASE
  return hipGetLastError();
}

}  // namespace zha
