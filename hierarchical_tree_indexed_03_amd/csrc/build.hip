// Tree build and append kernels.
//
// A node's summary, for each reference query r_j, is the tangent plane at r_j of the
// node's log attention mass f(q) = log sum_{k in span} exp(q.k / sqrt(d)) (news summary
// "Zyphra releases the ZHA sparse attention method", section "Building the tree"):
//   LSE_j = f(r_j),  s_j = grad f(r_j) * sqrt(d) = softmax-weighted mean key,
//   c_j   = LSE_j - r_j.s_j / sqrt(d).
// Level 1 is computed from the raw keys.  A parent's LSE_j is the logsumexp of its
// children's log masses at r_j and its s_j the children's s_j weighted by the softmax of
// those log masses (blog "Zyphra Hierarchical Attention", section "Building the tree":
// summaries are grouped and compressed again, recursively).  The children's log mass at
// r_j is their own LSE_j: each plane lower-bounds the convex f and plane j touches it at
// r_j, so the max over a child's planes evaluated at r_j is exactly its LSE_j.
//
// The leaf kernel builds every level whose span fits one tile of keys held in LDS; the
// logits r_j.k of the tile are one MFMA contraction (R x d by d x T).  Higher levels are
// built by the parent kernel from the level below.  Besides s and c the tree keeps LSE_j
// per node so parents and appends need no dot products: with A_j = LSE_j - c_j
// (= r_j.s_j / sqrt(d), the softmax-weighted mean logit) a parent has
// A_j = sum_c w_cj A_cj, and c_j = LSE_j - A_j.
#include "common.hpp"
#include "kernels.hpp"
#include "route_util.hpp"

namespace zha {

__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <typename TIn>
__device__ __forceinline__ float ld_f32(const TIn* p) { return to_f32(*p); }

// Logits Zs[t][j] = sigma * K[t] . r_j for the T tokens of the tile (MFMA, one 16-token
// row tile per step; columns are reference queries, padded to 16).
template <int D, int R, int T>
__device__ void tile_logits(const bf16_t* Ks, const bf16_t* refs_g, float sigma, int nt, float* Zs) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, kg = lane >> 4;
  bf16x8 rb[D / 32];
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (col < R) v = *(const uint4*)(refs_g + col * D + kk * 32 + kg * 8);
    rb[kk] = __builtin_bit_cast(bf16x8, v);
  }
  for (int rt = wave; rt < T / 16; rt += 4) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      uint4 v = *(const uint4*)(Ks + (rt * 16 + col) * D + kk * 32 + kg * 8);
      acc = mfma_bf16(__builtin_bit_cast(bf16x8, v), rb[kk], acc);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      int t = rt * 16 + kg * 4 + e;
      if (col < R) Zs[t * R + col] = t < nt ? sigma * acc[e] : -INFINITY;
    }
  }
}

template <int D, int R, int T>
__device__ void tile_logits(const float* Ks, const float* refs_g, float sigma, int nt, float* Zs) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, kg = lane >> 4;
  for (int rt = wave; rt < T / 16; rt += 4) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int kk = 0; kk < D / 4; ++kk) {
      float av = Ks[(rt * 16 + col) * D + kk * 4 + kg];
      float bv = col < R ? refs_g[col * D + kk * 4 + kg] : 0.f;
      acc = mfma_f32(av, bv, acc);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      int t = rt * 16 + kg * 4 + e;
      if (col < R) Zs[t * R + col] = t < nt ? sigma * acc[e] : -INFINITY;
    }
  }
}

__device__ __forceinline__ float4 ld4_f32(const float* p) { return *(const float4*)p; }
// MX FP4 of one element per lane, 32 consecutive elements in 32 consecutive lanes (element
// index e, lane e mod 32; all 32 lanes active): block amax by butterfly, codes gathered
// eight to a 32-bit word by the lane holding the word's first element.
__device__ __forceinline__ void store_fp4_lane(uint8_t* q, uint8_t* x, int64_t e, float v) {
  float am = fabsf(v);
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) am = fmaxf(am, __shfl_xor(am, o));
  const uint32_t sb = mx_scale_byte(am);
  uint32_t w = e2m1_code(v, sb) << (4 * (int)(e & 7));
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) w |= __shfl_xor(w, o);
  if ((e & 7) == 0) *(uint32_t*)(q + e / 2) = w;
  if ((e & 31) == 0) x[e / 32] = (uint8_t)sb;
}

// four floats as bfloat16 (nearest, ties to even) at an 8-byte aligned address
__device__ __forceinline__ void store_bf16x4(bf16_t* p, float4 v) {
  uint2 w;
  w.x = f2bf16_bits(v.x) | (f2bf16_bits(v.y) << 16);
  w.y = f2bf16_bits(v.z) | (f2bf16_bits(v.w) << 16);
  *(uint2*)p = w;
}
__device__ __forceinline__ float4 ld4_f32(const bf16_t* p) {
  uint2 v = *(const uint2*)p;
  return make_float4(bf16_bits_to_f32(v.x & 0xffffu), bf16_bits_to_f32(v.x >> 16),
                     bf16_bits_to_f32(v.y & 0xffffu), bf16_bits_to_f32(v.y >> 16));
}

template <typename TIn, int D, int R, int T>
__global__ __launch_bounds__(256) void build_tile_kernel(BuildArgs a) {
  constexpr int NT = 256;
  __shared__ __align__(16) TIn Ks[T * D];
  __shared__ float Zs[T * R];
  __shared__ float Ws[T * R];
  __shared__ float Ls[T * R];
  __shared__ float As[T * R];
  // s of the last in-tile level, for the next level's recursion (R < 8 path)
  constexpr int SR_HALF = R < 8 ? 2048 : 4;
  // bf16 keys, R = 16, 128-token tiles: the weighted means of levels 1 and 2 by the register
  // path (a thread per (node, 4 columns) sums the node's keys for all R planes), which issues
  // far fewer instructions than one MFMA item per (node, 16 columns) over b or b^2 tokens;
  // the levels above keep the MFMA items (measured: 0.79 ms against 1.03 ms for the deep
  // tree at 256K, and 0.84 ms with every in-tile level on the register path)
  constexpr bool L12_REG = R == 16 && sizeof(TIn) == 2 && T == 128;
  __shared__ __align__(16) float Sr[2 * SR_HALF];

  const int kv = blockIdx.y;
  // a new tree: the append's cached sibling aggregates no longer hold
  if (blockIdx.x == 0 && threadIdx.x <= MAXL) a.dev.sibkey[(int64_t)kv * (MAXL + 1) + threadIdx.x] = -1;
  const TIn* Rg = (const TIn*)a.refs + (int64_t)kv * R * D;
  const int64_t ntiles = (a.N + T - 1) / T;

  // Persistent workgroups: tiles blockIdx.x, + gridDim.x, ...; the next tile's keys are
  // loaded into registers while the current tile is summarised.
  constexpr int CH = 16 / sizeof(TIn);
  constexpr int KPT = T * D / CH / NT;        // 16-byte key pieces per thread per tile
  uint4 kreg[KPT];
  auto load_tile = [&](int64_t tile) {
    const int64_t tt0 = tile * T;
    const int ntt = (int)min((int64_t)T, a.N - tt0);
    const TIn* Kg = (const TIn*)a.K + ((int64_t)kv * a.cap + tt0) * D;
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int i = threadIdx.x + u * NT;
      const int row = (i * CH) / D;
      kreg[u] = row < ntt ? *(const uint4*)(Kg + (int64_t)i * CH) : make_uint4(0, 0, 0, 0);
    }
  };
  // tiles a.tile0 .. ntiles-1 (a.tile0 > 0: the tail of a multi-token append)
  if (a.tile0 + (int64_t)blockIdx.x < ntiles) load_tile(a.tile0 + blockIdx.x);
  for (int64_t tile = a.tile0 + blockIdx.x; tile < ntiles; tile += gridDim.x) {
  const int64_t t0 = tile * T;
  const int nt = (int)min((int64_t)T, a.N - t0);
#pragma unroll
  for (int u = 0; u < KPT; ++u) *(uint4*)(Ks + (threadIdx.x + u * NT) * CH) = kreg[u];
  __syncthreads();
  if (tile + gridDim.x < ntiles) load_tile(tile + gridDim.x);
  tile_logits<D, R, T>(Ks, Rg, a.sigma, nt, Zs);
  __syncthreads();

  // LSE_j and A_j per node, level by level (children before parents).
  int off[MAXL + 2];
  off[1] = 0;
  int64_t bv = 1;
  for (int v = 1; v <= a.m; ++v) {
    const int64_t bprev = bv;
    bv *= a.b;
    off[v + 1] = off[v] + (int)(T / bv) * R;
    const int nv = (int)(T / bv);
    const int nexist = (int)((nt + bv - 1) / bv);
    const int nprev_exist = (int)((nt + bprev - 1) / bprev);
    // P threads per (node, plane) when there are fewer pairs than threads (wide nodes), the
    // P partial max / sums combined across the group's lanes in a fixed order
    int P = 1;
    while (P < 64 && P * 2 * nv * R <= NT) P *= 2;
    const int sub = threadIdx.x % P;
    for (int idx = threadIdx.x / P; idx < nv * R; idx += NT / P) {
      const int node = idx / R, j = idx % R;
      if (node >= nexist) continue;   // the whole group skips together
      const float* src;   // the node's children: the tokens' logits, or the level below
      const float* Ac = nullptr;
      int cb, ce;
      if (v == 1) {
        cb = node * a.b;
        ce = min(cb + a.b, nt);
        src = Zs;
      } else {
        cb = node * a.b;
        ce = min(cb + a.b, nprev_exist);
        src = Ls + off[v - 1];
        Ac = As + off[v - 1];
      }
      float mx = -INFINITY, sum = 0.f, A = 0.f;
      for (int c = cb + sub; c < ce; c += P) mx = fmaxf(mx, src[c * R + j]);
      for (int o = P / 2; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
      for (int c = cb + sub; c < ce; c += P) sum += expf(src[c * R + j] - mx);
      for (int o = P / 2; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
      const float lse = mx + logf(sum);
      for (int c = cb + sub; c < ce; c += P)
        A += expf(src[c * R + j] - lse) * (v == 1 ? src[c * R + j] : Ac[c * R + j]);
      for (int o = P / 2; o > 0; o >>= 1) A += __shfl_xor(A, o);
      if (sub == 0) {
        Ls[off[v] + idx] = lse;
        As[off[v] + idx] = A;
        const int64_t gnode = t0 / bv + node;
        const int64_t gi = ((int64_t)kv * a.dev.ncap[v] + gnode) * R + j;
        a.dev.c[v][gi] = lse - A;
        a.dev.lse[v][gi] = lse;
      }
    }
    __syncthreads();
  }

  // Weighted-mean keys s_j of every node of every in-tile level: from the keys (MFMA path,
  // and level 1), or from the level below (VALU path, see there).
  bv = 1;
  bool recur_ok = false;
  for (int v = 1; v <= a.m; ++v) {
    bv *= a.b;
    const int nexist = (int)((nt + bv - 1) / bv);
    for (int idx = threadIdx.x; idx < T * R; idx += NT) {
      const int t = idx / R, j = idx % R;
      Ws[idx] = t < nt ? expf(Zs[idx] - Ls[off[v] + (int)(t / bv) * R + j]) : 0.f;
    }
    __syncthreads();
    if (v == 1 && a.dev.w1) {
      // token weights of the level-1 planes, [node][j][token in block] (zero past the data)
      const int b = a.b;
      for (int idx = threadIdx.x; idx < nexist * R * b; idx += NT) {
        const int node = idx / (R * b), j = (idx / b) % R, k = idx % b;
        const int t = node * b + k;
        a.dev.w1[((int64_t)kv * a.dev.ncap[1] + t0 / b + node) * R * b + j * b + k] = t < nt ? Ws[t * R + j] : 0.f;
      }
    }
    if (R >= 8 && !(L12_REG && v <= 2)) {
      const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
      const int col = lane & 15, kg = lane >> 4;
      const int items = nexist * (D / 16);
      for (int it = wave; it < items; it += 4) {
        const int node = it / (D / 16), n16 = it % (D / 16);
        const int ts = node * (int)bv;
        const int te = min(ts + (int)bv, nt);
        // four independent accumulation chains over 16-token groups (their LDS loads issued
        // together), then the tail 4 tokens at a time; summed chain by chain at the end
        f32x4 acc4[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) acc4[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        int st = ts;
        for (; st + 16 <= te; st += 16) {
          float w[4], kvv[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int t = st + 4 * u + kg;
            w[u] = col < R ? Ws[t * R + col] : 0.f;
            kvv[u] = ld_f32(Ks + t * D + n16 * 16 + col);
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) acc4[u] = mfma_f32(w[u], kvv[u], acc4[u]);
        }
        for (; st < te; st += 4) {
          const int t = st + kg;
          const bool ok = t < te;
          float w = (ok && col < R) ? Ws[t * R + col] : 0.f;
          float kvv = ok ? ld_f32(Ks + t * D + n16 * 16 + col) : 0.f;
          acc4[0] = mfma_f32(w, kvv, acc4[0]);
        }
        const f32x4 acc = ((acc4[0] + acc4[1]) + acc4[2]) + acc4[3];
        const int64_t gnode = t0 / bv + node;
        const int64_t so = (((int64_t)kv * a.dev.ncap[v] + gnode) * R) * D + n16 * 16 + col;
        float* sg = a.dev.s[v] + so;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = kg * 4 + e;
          if (j < R) sg[(int64_t)j * D] = acc[e];
        }
        if (a.dev.sq[v]) {
          uint16_t* qg = (uint16_t*)a.dev.sq[v] + so;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int j = kg * 4 + e;
            if (j < R) qg[(int64_t)j * D] = (uint16_t)f2bf16_bits(acc[e]);
          }
        }
      }
    } else {
      // level 1 from the keys; a higher in-tile level from the level below while that level
      // fits the LDS buffer (s_parent = sum over children of exp(LSE_c - LSE_parent) s_c),
      // else from the keys of its whole span
      const int nprev = v == 1 ? 0 : (int)((nt + bv / a.b - 1) / (bv / a.b));
      const bool from_children = v > 1 && nprev * R * D <= SR_HALF && recur_ok;
      const float* Sprev = Sr + ((v - 1) & 1) * SR_HALF;
      float* Scur = Sr + (v & 1) * SR_HALF;
      const bool keep_cur = nexist * R * D <= SR_HALF;
      const int items = nexist * (D / 4);
      for (int it = threadIdx.x; it < items; it += NT) {
        const int node = it / (D / 4), dc = it % (D / 4);
        float4 acc[R];
#pragma unroll
        for (int j = 0; j < R; ++j) acc[j] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (from_children) {
          const int cb = node * a.b, ce = min(cb + a.b, nprev);
          for (int ch = cb; ch < ce; ++ch) {
#pragma unroll
            for (int j = 0; j < R; ++j) {
              const float w = expf(Ls[off[v - 1] + ch * R + j] - Ls[off[v] + node * R + j]);
              const float4 s4 = *(const float4*)(Sprev + (ch * R + j) * D + dc * 4);
              acc[j].x += w * s4.x; acc[j].y += w * s4.y; acc[j].z += w * s4.z; acc[j].w += w * s4.w;
            }
          }
        } else {
          const int ts = node * (int)bv, te = min(ts + (int)bv, nt);
          for (int t = ts; t < te; ++t) {
            float4 k4 = ld4_f32(Ks + t * D + dc * 4);
#pragma unroll
            for (int j = 0; j < R; ++j) {
              float w = Ws[t * R + j];
              acc[j].x += w * k4.x; acc[j].y += w * k4.y; acc[j].z += w * k4.z; acc[j].w += w * k4.w;
            }
          }
        }
        const int64_t gnode = t0 / bv + node;
        const int64_t so = (((int64_t)kv * a.dev.ncap[v] + gnode) * R) * D + dc * 4;
        float* sg = a.dev.s[v] + so;
#pragma unroll
        for (int j = 0; j < R; ++j) *(float4*)(sg + (int64_t)j * D) = acc[j];
        if (a.dev.sq[v])
#pragma unroll
          for (int j = 0; j < R; ++j) store_bf16x4(a.dev.sq[v] + so + (int64_t)j * D, acc[j]);
        if (keep_cur)
#pragma unroll
          for (int j = 0; j < R; ++j) *(float4*)(Scur + (node * R + j) * D + dc * 4) = acc[j];
      }
      recur_ok = keep_cur;
    }
    __syncthreads();
  }
  }
}

// One parent from its children at level v-1.  Work of PPB parents per workgroup.
template <int D, int R>
__device__ void parent_nodes(const Dev& dev, int v, int kv, int b, int64_t p0, int np, int64_t nchild,
                             float* Lp, float* Wp) {
  constexpr int NT = 256;
  const int64_t ccap = dev.ncap[v - 1], pcap = dev.ncap[v];
  const float* lse_c = dev.lse[v - 1] + (int64_t)kv * ccap * R;
  const float* c_c = dev.c[v - 1] + (int64_t)kv * ccap * R;
  for (int idx = threadIdx.x; idx < np * R; idx += NT) {
    const int p = idx / R, j = idx % R;
    const int64_t gp = p0 + p;
    const int64_t cb = gp * b, ce = min(cb + b, nchild);
    float mx = -INFINITY, sum = 0.f, A = 0.f;
    for (int64_t ch = cb; ch < ce; ++ch) mx = fmaxf(mx, lse_c[ch * R + j]);
    for (int64_t ch = cb; ch < ce; ++ch) sum += expf(lse_c[ch * R + j] - mx);
    const float lse = mx + logf(sum);
    for (int64_t ch = cb; ch < ce; ++ch) {
      const float lc = lse_c[ch * R + j];
      const float w = expf(lc - lse);
      Wp[(p * b + (int)(ch - cb)) * R + j] = w;
      A += w * (lc - c_c[ch * R + j]);
    }
    for (int64_t ch = ce; ch < cb + b; ++ch) Wp[(p * b + (int)(ch - cb)) * R + j] = 0.f;
    Lp[idx] = lse;
    const int64_t gi = ((int64_t)kv * pcap + gp) * R + j;
    dev.c[v][gi] = lse - A;
    dev.lse[v][gi] = lse;
  }
  __syncthreads();
  const float* s_c = dev.s[v - 1] + (int64_t)kv * ccap * R * D;
  for (int it = threadIdx.x; it < np * R * (D / 4); it += NT) {
    const int p = it / (R * (D / 4));
    const int rem = it % (R * (D / 4));
    const int j = rem / (D / 4), dc = rem % (D / 4);
    const int64_t gp = p0 + p;
    const int64_t cb = gp * b, ce = min(cb + b, nchild);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int64_t ch = cb; ch < ce; ++ch) {
      const float w = Wp[(p * b + (int)(ch - cb)) * R + j];
      const float4 s4 = *(const float4*)(s_c + (ch * R + j) * D + dc * 4);
      acc.x += w * s4.x; acc.y += w * s4.y; acc.z += w * s4.z; acc.w += w * s4.w;
    }
    const int64_t so = (((int64_t)kv * pcap + gp) * R + j) * D + dc * 4;
    *(float4*)(dev.s[v] + so) = acc;
    if (dev.sq[v]) store_bf16x4(dev.sq[v] + so, acc);
  }
}

template <int D, int R>
constexpr int parents_per_block() {
  return (R * (D / 4)) >= 256 ? 1 : 256 / (R * (D / 4));
}

template <int D, int R>
__global__ __launch_bounds__(256) void build_parent_kernel(ParentArgs a) {
  constexpr int PPB = parents_per_block<D, R>();
  __shared__ float Lp[PPB * R];
  __shared__ float Wp[PPB * 256 * R];
  const int kv = blockIdx.y;
  const int64_t p0 = a.first + (int64_t)blockIdx.x * PPB;
  const int np = (int)min((int64_t)PPB, a.nparent - p0);
  if (np <= 0) return;
  parent_nodes<D, R>(a.dev, a.level, kv, a.b, p0, np, a.nchild, Lp, Wp);
}

// b^e saturated at 2^62 (spans above every token count)
__device__ __forceinline__ int64_t ipow64(int64_t b, int e) {
  int64_t r = 1;
  for (int i = 0; i < e; ++i) {
    if (r > ((int64_t)1 << 62) / b) return (int64_t)1 << 62;
    r *= b;
  }
  return r;
}

// Append one token per KV head and refresh the rightmost node of every level.
//
// The new token only changes the rightmost node of each level.  Level 1 is updated in place:
// with z_j = r_j.k_new / sqrt(d), LSE' = logaddexp(LSE, z_j), the old softmax weights scale
// by exp(LSE - LSE') and the new key enters with weight exp(z_j - LSE'), so s_j, A_j and the
// stored token weights follow with no pass over the block's keys.  A parent is the
// logsumexp / softmax-weighted mean over its children: its complete children (all but the
// rightmost) are folded into one aggregate (LSE, A, s), kept in the workspace and rebuilt
// only when that set of children changes (once every b^(v-1) tokens at level v); the
// rightmost child is the node just refreshed one level down.  With the aggregates loaded,
// each thread carries its own (plane, dim) elements up through every level with no barrier.
// One workgroup per KV head.
template <typename TIn, int D, int R>
__global__ __launch_bounds__(1024) void append_kernel(AppendArgs a) {
  constexpr int NT = 1024;
  constexpr int NW = NT / 64;
  constexpr int RD = R * D;
  constexpr int RS = SIB_LEVEL(R, D);         // aggregate per level: [j][LSE, A, s(D)], padded
  __shared__ __align__(16) float Agg[(MAXL - 1) * RS];
  __shared__ float zl[R], Lo[R], Ao[R];     // new-token logits; old level-1 LSE and A
  __shared__ int64_t keyl[MAXL];              // per level v (index v-2): first child * 256 + count
  __shared__ int64_t pvl[MAXL];               // per level v (index v-2): the refreshed node
  __shared__ float Cf[MAXL][R][2];            // per level (index v-1), plane: weights of old, new
  __shared__ int stale[MAXL];
  const int kv = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t n = a.N;        // index of the new token
  const int b = a.b, L = a.levels;
  TIn* Kc = (TIn*)a.K + (int64_t)kv * a.cap * D;
  TIn* Vc = (TIn*)a.V + (int64_t)kv * a.cap * D;
  const TIn* kn = (const TIn*)a.k_new + (int64_t)kv * a.new_stride;
  const TIn* vn = (const TIn*)a.v_new + (int64_t)kv * a.new_stride;
  for (int i = tid; i < D; i += NT) {
    Kc[n * D + i] = kn[i];
    Vc[n * D + i] = vn[i];
  }
  const int64_t n1 = n / b;
  const int k1 = (int)(n - n1 * b);           // position of the new token in its block
  const int64_t g1 = (int64_t)kv * a.dev.ncap[1] + n1;
  float* sib = a.dev.sib + (int64_t)kv * SIB_STRIDE(R, D);
  int64_t* sibkey = a.dev.sibkey + (int64_t)kv * (MAXL + 1);
  // cached aggregates of every level, and whether their set of children still holds
  if (tid < L - 1) {
    const int v = tid + 2;
    const int64_t last = n / ipow64(b, v - 1), pv = n / ipow64(b, v), c0 = pv * b;
    const int64_t key = c0 * 256 + (last - c0);
    keyl[tid] = key;
    pvl[tid] = pv;
    stale[tid] = sibkey[v] != key;
  }
  {   // levels 2..L, float4 loads all issued together
    constexpr int U = 8;
    const int tot4 = (L - 1) * RS / 4;
    const float4* src = (const float4*)(sib + 2 * RS);
    for (int i0 = tid; i0 < tot4; i0 += NT * U) {
      float4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = i0 + u * NT < tot4 ? src[i0 + u * NT] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (i0 + u * NT < tot4) ((float4*)Agg)[i0 + u * NT] = v[u];
    }
  }
  // the old level-1 s of this thread's elements
  constexpr int IT = (RD + NT - 1) / NT;
  float sold[IT];
#pragma unroll
  for (int u = 0; u < IT; ++u) {
    const int i = tid + u * NT;
    sold[u] = (i < RD && k1) ? a.dev.s[1][g1 * RD + i] : 0.f;
  }
  if (tid < R) {
    const float lo = k1 ? a.dev.lse[1][g1 * R + tid] : -INFINITY;
    Lo[tid] = lo;
    Ao[tid] = k1 ? lo - a.dev.c[1][g1 * R + tid] : 0.f;
  }
  // z_j = sigma r_j . k_new, one wave per reference query
  const TIn* Rg = (const TIn*)a.refs + (int64_t)kv * R * D;
  for (int j = wave; j < R; j += NW) {
    float part = 0.f;
    for (int i = lane; i < D; i += 64) part += to_f32(Rg[j * D + i]) * to_f32(kn[i]);
    for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off);
    if (lane == 0) zl[j] = a.sigma * part;
  }
  __syncthreads();
  // rebuild the aggregates whose set of children changed (all threads, one level at a time)
  for (int vi = 0; vi < L - 1; ++vi) {
    if (!stale[vi]) continue;     // block-uniform
    const int v = vi + 2;
    const int64_t c0 = keyl[vi] >> 8;
    const int nsib = (int)(keyl[vi] & 255);
    const int64_t ccap = a.dev.ncap[v - 1];
    const float* lse_c = a.dev.lse[v - 1] + ((int64_t)kv * ccap + c0) * R;
    const float* c_c = a.dev.c[v - 1] + ((int64_t)kv * ccap + c0) * R;
    const float* s_c = a.dev.s[v - 1] + ((int64_t)kv * ccap + c0) * RD;
    float* ag = Agg + vi * RS;
    for (int i = tid; i < R * (D + 2); i += NT) {
      const int j = i / (D + 2), k = i % (D + 2);
      float m = -INFINITY;
      for (int c = 0; c < nsib; ++c) m = fmaxf(m, lse_c[c * R + j]);
      float sum = 0.f, acc = 0.f;
      for (int c = 0; c < nsib; ++c) {
        const float lc = lse_c[c * R + j];
        const float e = expf(lc - m);
        sum += e;
        acc += e * (k == 0 ? 0.f : k == 1 ? lc - c_c[c * R + j] : s_c[(int64_t)c * RD + j * D + k - 2]);
      }
      const float val = nsib == 0 ? (k == 0 ? -INFINITY : 0.f) : (k == 0 ? m + logf(sum) : acc / sum);
      ag[i] = val;
      sib[(int64_t)v * RS + i] = val;
    }
    __syncthreads();
    if (tid == 0) sibkey[v] = keyl[vi];
  }
  // ---- per plane j, the chain of merges from level 1 to the top (one thread per plane):
  // LSE and A of every refreshed node, and the weights (old, new) each level applies to s
  if (tid < R) {
    const int j = tid;
    const float z = zl[j];
    float lse, A, al, be;
    if (k1 == 0) {
      lse = z; A = z; al = 0.f; be = 1.f;
    } else {
      const float lo = Lo[j];
      const float m = fmaxf(lo, z);
      lse = m + logf(expf(lo - m) + expf(z - m));
      al = expf(lo - lse);
      be = expf(z - lse);
      A = al * Ao[j] + be * z;
    }
    Cf[0][j][0] = al; Cf[0][j][1] = be;
    a.dev.lse[1][g1 * R + j] = lse;
    a.dev.c[1][g1 * R + j] = lse - A;
    for (int v = 2; v <= L; ++v) {
      const float* ag = Agg + (v - 2) * RS + j * (D + 2);
      const float ls = ag[0];
      float wa = 0.f, wb = 1.f;
      if (ls != -INFINITY) {
        const float m = fmaxf(ls, lse);
        const float lp = m + logf(expf(ls - m) + expf(lse - m));
        wa = expf(ls - lp);
        wb = expf(lse - lp);
        A = wa * ag[1] + wb * A;
        lse = lp;
      }
      Cf[v - 1][j][0] = wa; Cf[v - 1][j][1] = wb;
      const int64_t gp = (int64_t)kv * a.dev.ncap[v] + pvl[v - 2];
      a.dev.lse[v][gp * R + j] = lse;
      a.dev.c[v][gp * R + j] = lse - A;
    }
  }
  __syncthreads();
  // ---- s of every refreshed node: each thread carries its (plane j, dim d) elements up
#pragma unroll
  for (int u = 0; u < IT; ++u) {
    const int i = tid + u * NT;
    if (i >= RD) break;
    const int j = i / D, d = i % D;
    const float kd = to_f32(kn[d]);
    float sv = Cf[0][j][0] * sold[u] + Cf[0][j][1] * kd;
    a.dev.s[1][g1 * RD + i] = sv;
    if (a.dev.sq[1]) a.dev.sq[1][g1 * RD + i].bits = (uint16_t)f2bf16_bits(sv);
    if (a.dev.s4[1]) store_fp4_lane(a.dev.s4[1], a.dev.s4x[1], g1 * RD + i, sv);
    for (int v = 2; v <= L; ++v) {
      sv = Cf[v - 1][j][0] * Agg[(v - 2) * RS + j * (D + 2) + 2 + d] + Cf[v - 1][j][1] * sv;
      const int64_t si = ((int64_t)kv * a.dev.ncap[v] + pvl[v - 2]) * RD + i;
      a.dev.s[v][si] = sv;
      if (a.dev.sq[v]) a.dev.sq[v][si].bits = (uint16_t)f2bf16_bits(sv);
      if (a.dev.s4[v]) store_fp4_lane(a.dev.s4[v], a.dev.s4x[v], si, sv);
    }
  }
  // token weights of the level-1 planes (key-form scoring): old weights scale by
  // exp(LSE - LSE'), the new token's weight is exp(z_j - LSE'), later slots stay zero
  if (a.dev.w1) {
    float* wg = a.dev.w1 + g1 * R * b;
    for (int i = tid; i < R * b; i += NT) {
      const int j = i / b, k = i % b;
      float w = 0.f;
      if (k < k1) w = Cf[0][j][0] * wg[i];
      else if (k == k1) w = Cf[0][j][1];
      wg[i] = w;
    }
  }
}

// ---------------------------------------------------------------- host launchers
// One wave of resident workgroups per launch, spread over the KV heads; each strides over
// its tiles.
template <typename TIn, int D, int R, int T>
static void launch_build_tiles(const BuildArgs& a, int64_t ntiles, int hkv, hipStream_t st) {
  static const int per_cu = resident_per_cu(build_tile_kernel<TIn, D, R, T>, 256);
  int64_t x = (int64_t)per_cu * device_cus() / hkv;
  if (x > ntiles - a.tile0) x = ntiles - a.tile0;
  if (x < 1) x = 1;
  hipLaunchKernelGGL((build_tile_kernel<TIn, D, R, T>), dim3((unsigned)x, (unsigned)hkv), dim3(256), 0, st, a);
}

template <typename TIn, int D, int R>
static hipError_t launch_build_d(const BuildArgs& a, int64_t ntiles, int hkv, int T, hipStream_t st) {
  if (T == 128) {
    launch_build_tiles<TIn, D, R, 128>(a, ntiles, hkv, st);
  } else {
    // 256-token tiles (blocks of more than 128 keys) only where the tile fits in LDS
    if constexpr (sizeof(TIn) * 256 * D + 16 * 256 * R <= 160 * 1024)
      launch_build_tiles<TIn, D, R, 256>(a, ntiles, hkv, st);
    else
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename TIn>
static hipError_t launch_build_t(const BuildArgs& a, int D, int R, int64_t ntiles, int hkv, int T, hipStream_t st) {
#define ZHA_CASE(DD, RR) if (D == DD && R == RR) return launch_build_d<TIn, DD, RR>(a, ntiles, hkv, T, st);
  ZHA_CASE(64, 1) ZHA_CASE(64, 2) ZHA_CASE(64, 4) ZHA_CASE(64, 8) ZHA_CASE(64, 16)
  ZHA_CASE(128, 1) ZHA_CASE(128, 2) ZHA_CASE(128, 4) ZHA_CASE(128, 8) ZHA_CASE(128, 16)
#undef ZHA_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_build_tile(const BuildArgs& a, bool bf16, int D, int R, int64_t ntiles, int hkv, int T,
                             hipStream_t st) {
  return bf16 ? launch_build_t<bf16_t>(a, D, R, ntiles, hkv, T, st)
              : launch_build_t<float>(a, D, R, ntiles, hkv, T, st);
}

hipError_t launch_build_parent(const ParentArgs& a, int D, int R, int hkv, hipStream_t st) {
#define ZHA_CASE(DD, RR)                                                                  \
  if (D == DD && R == RR) {                                                               \
    constexpr int PPB = parents_per_block<DD, RR>();                                      \
    dim3 grid((unsigned)((a.nparent - a.first + PPB - 1) / PPB), (unsigned)hkv);           \
    hipLaunchKernelGGL((build_parent_kernel<DD, RR>), grid, dim3(256), 0, st, a);         \
    return hipGetLastError();                                                             \
  }
  ZHA_CASE(64, 1) ZHA_CASE(64, 2) ZHA_CASE(64, 4) ZHA_CASE(64, 8) ZHA_CASE(64, 16)
  ZHA_CASE(128, 1) ZHA_CASE(128, 2) ZHA_CASE(128, 4) ZHA_CASE(128, 8) ZHA_CASE(128, 16)
#undef ZHA_CASE
  return hipErrorInvalidValue;
}

// MX FP4 copy of one level's s: a thread per 4 consecutive elements, 8 threads per
// 32-element block (amax by 3 butterfly steps; a block's threads run the loop together);
// each thread stores its 16 code bits, the block's first thread the scale byte.
template <int D, int R>
__global__ __launch_bounds__(256) void quantise_fp4_kernel(QuantArgs a) {
  const int kv = blockIdx.y, v = a.level;
  const int64_t cap = a.dev.ncap[v];
  const int64_t items = a.nnode * R * (D / 4);
  const float* S = a.dev.s[v] + (int64_t)kv * cap * R * D;
  uint8_t* Q = a.dev.s4[v] + (int64_t)kv * cap * R * D / 2;
  uint8_t* X = a.dev.s4x[v] + (int64_t)kv * cap * R * D / 32;
  for (int64_t it = a.first * R * (D / 4) + (int64_t)blockIdx.x * 256 + threadIdx.x; it < items;
       it += (int64_t)gridDim.x * 256) {
    const float4 x = *(const float4*)(S + it * 4);
    float am = fmaxf(fmaxf(fabsf(x.x), fabsf(x.y)), fmaxf(fabsf(x.z), fabsf(x.w)));
    am = fmaxf(am, __shfl_xor(am, 1));
    am = fmaxf(am, __shfl_xor(am, 2));
    am = fmaxf(am, __shfl_xor(am, 4));
    const uint32_t sb = mx_scale_byte(am);
    const uint32_t c = e2m1_code(x.x, sb) | (e2m1_code(x.y, sb) << 4) | (e2m1_code(x.z, sb) << 8) |
                       (e2m1_code(x.w, sb) << 12);
    *(uint16_t*)(Q + it * 2) = (uint16_t)c;
    if ((it & 7) == 0) X[it / 8] = (uint8_t)sb;
  }
}

hipError_t launch_quantise_fp4(const QuantArgs& a, int D, int R, int hkv, hipStream_t st) {
  const int64_t items = (a.nnode - a.first) * R * (D / 4);
  int64_t x = (items + 255) / 256;
  if (x > 4096) x = 4096;
  if (x < 1) x = 1;
#define ZHA_CASE(DD, RR)                                                                               \
  if (D == DD && R == RR) {                                                                            \
    hipLaunchKernelGGL((quantise_fp4_kernel<DD, RR>), dim3((unsigned)x, (unsigned)hkv), dim3(256), 0, st, a); \
    return hipGetLastError();                                                                          \
  }
  ZHA_CASE(64, 1) ZHA_CASE(64, 2) ZHA_CASE(64, 4) ZHA_CASE(64, 8) ZHA_CASE(64, 16)
  ZHA_CASE(128, 1) ZHA_CASE(128, 2) ZHA_CASE(128, 4) ZHA_CASE(128, 8) ZHA_CASE(128, 16)
#undef ZHA_CASE
  return hipErrorInvalidValue;
}

template <typename TIn>
static hipError_t launch_append_t(const AppendArgs& a, int D, int R, int hkv, hipStream_t st) {
#define ZHA_CASE(DD, RR)                                                                   \
  if (D == DD && R == RR) {                                                                \
    hipLaunchKernelGGL((append_kernel<TIn, DD, RR>), dim3(hkv), dim3(1024), 0, st, a);     \
    return hipGetLastError();                                                              \
  }
  ZHA_CASE(64, 1) ZHA_CASE(64, 2) ZHA_CASE(64, 4) ZHA_CASE(64, 8) ZHA_CASE(64, 16)
  ZHA_CASE(128, 1) ZHA_CASE(128, 2) ZHA_CASE(128, 4) ZHA_CASE(128, 8) ZHA_CASE(128, 16)
#undef ZHA_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_append(const AppendArgs& a, bool bf16, int D, int R, int hkv, hipStream_t st) {
  return bf16 ? launch_append_t<bf16_t>(a, D, R, hkv, st) : launch_append_t<float>(a, D, R, hkv, st);
}

}  // namespace zha
