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

  const int kv = blockIdx.y;
  const int64_t t0 = (int64_t)blockIdx.x * T;
  const int nt = (int)min((int64_t)T, a.N - t0);
  const TIn* Kg = (const TIn*)a.K + ((int64_t)kv * a.cap + t0) * D;
  const TIn* Rg = (const TIn*)a.refs + (int64_t)kv * R * D;

  constexpr int CH = 16 / sizeof(TIn);
  for (int i = threadIdx.x; i < T * D / CH; i += NT) {
    int row = (i * CH) / D;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (row < nt) v = *(const uint4*)(Kg + (int64_t)i * CH);
    *(uint4*)(Ks + i * CH) = v;
  }
  __syncthreads();
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
    for (int idx = threadIdx.x; idx < nv * R; idx += NT) {
      const int node = idx / R, j = idx % R;
      if (node >= nexist) continue;
      float mx = -INFINITY, sum = 0.f, lse, A = 0.f;
      if (v == 1) {
        const int tb = node * a.b, te = min(tb + a.b, nt);
        for (int t = tb; t < te; ++t) mx = fmaxf(mx, Zs[t * R + j]);
        for (int t = tb; t < te; ++t) sum += expf(Zs[t * R + j] - mx);
        lse = mx + logf(sum);
        for (int t = tb; t < te; ++t) A += expf(Zs[t * R + j] - lse) * Zs[t * R + j];
      } else {
        const int cb = node * a.b, ce = min(cb + a.b, nprev_exist);
        const float* Lc = Ls + off[v - 1];
        const float* Ac = As + off[v - 1];
        for (int ch = cb; ch < ce; ++ch) mx = fmaxf(mx, Lc[ch * R + j]);
        for (int ch = cb; ch < ce; ++ch) sum += expf(Lc[ch * R + j] - mx);
        lse = mx + logf(sum);
        for (int ch = cb; ch < ce; ++ch) A += expf(Lc[ch * R + j] - lse) * Ac[ch * R + j];
      }
      Ls[off[v] + idx] = lse;
      As[off[v] + idx] = A;
      const int64_t gnode = t0 / bv + node;
      const int64_t gi = ((int64_t)kv * a.dev.ncap[v] + gnode) * R + j;
      a.dev.c[v][gi] = lse - A;
      a.dev.lse[v][gi] = lse;
    }
    __syncthreads();
  }

  // Weighted-mean keys s_j of every node of every in-tile level, straight from the keys.
  bv = 1;
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
    if constexpr (R >= 8) {
      const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
      const int col = lane & 15, kg = lane >> 4;
      const int items = nexist * (D / 16);
      for (int it = wave; it < items; it += 4) {
        const int node = it / (D / 16), n16 = it % (D / 16);
        const int ts = node * (int)bv;
        const int te = min(ts + (int)bv, nt);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int st = ts; st < te; st += 4) {
          const int t = st + kg;
          const bool ok = t < te;
          float w = (ok && col < R) ? Ws[t * R + col] : 0.f;
          float kvv = ok ? ld_f32(Ks + t * D + n16 * 16 + col) : 0.f;
          acc = mfma_f32(w, kvv, acc);
        }
        const int64_t gnode = t0 / bv + node;
        float* sg = a.dev.s[v] + (((int64_t)kv * a.dev.ncap[v] + gnode) * R) * D + n16 * 16 + col;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = kg * 4 + e;
          if (j < R) sg[(int64_t)j * D] = acc[e];
        }
      }
    } else {
      const int items = nexist * (D / 4);
      for (int it = threadIdx.x; it < items; it += NT) {
        const int node = it / (D / 4), dc = it % (D / 4);
        const int ts = node * (int)bv, te = min(ts + (int)bv, nt);
        float4 acc[R];
#pragma unroll
        for (int j = 0; j < R; ++j) acc[j] = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int t = ts; t < te; ++t) {
          float4 k4 = ld4_f32(Ks + t * D + dc * 4);
#pragma unroll
          for (int j = 0; j < R; ++j) {
            float w = Ws[t * R + j];
            acc[j].x += w * k4.x; acc[j].y += w * k4.y; acc[j].z += w * k4.z; acc[j].w += w * k4.w;
          }
        }
        const int64_t gnode = t0 / bv + node;
        float* sg = a.dev.s[v] + (((int64_t)kv * a.dev.ncap[v] + gnode) * R) * D + dc * 4;
#pragma unroll
        for (int j = 0; j < R; ++j) *(float4*)(sg + (int64_t)j * D) = acc[j];
      }
    }
    __syncthreads();
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
    *(float4*)(dev.s[v] + (((int64_t)kv * pcap + gp) * R + j) * D + dc * 4) = acc;
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
  const int64_t p0 = (int64_t)blockIdx.x * PPB;
  const int np = (int)min((int64_t)PPB, a.nparent - p0);
  if (np <= 0) return;
  parent_nodes<D, R>(a.dev, a.level, kv, a.b, p0, np, a.nchild, Lp, Wp);
}

// Append one token per KV head and refresh the rightmost node of every level.
template <typename TIn, int D, int R>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  constexpr int NT = 256;
  __shared__ float Zs[256 * R];
  __shared__ float Lj[R];
  __shared__ float Lp[R];
  __shared__ float Wp[256 * R];
  const int kv = blockIdx.x;
  const int64_t n = a.N;  // index of the new token
  TIn* Kc = (TIn*)a.K + (int64_t)kv * a.cap * D;
  TIn* Vc = (TIn*)a.V + (int64_t)kv * a.cap * D;
  const TIn* kn = (const TIn*)a.k_new + (int64_t)kv * D;
  const TIn* vn = (const TIn*)a.v_new + (int64_t)kv * D;
  for (int i = threadIdx.x; i < D; i += NT) {
    Kc[n * D + i] = kn[i];
    Vc[n * D + i] = vn[i];
  }
  // level 1: block n1 holds tokens [n1*b, n] after the append
  const int64_t n1 = n / a.b;
  const int64_t tb = n1 * a.b;
  const int nt = (int)(n - tb + 1);
  const TIn* Rg = (const TIn*)a.refs + (int64_t)kv * R * D;
  for (int idx = threadIdx.x; idx < nt * R; idx += NT) {
    const int t = idx / R, j = idx % R;
    const TIn* kr = (tb + t == n) ? kn : Kc + (tb + t) * D;
    float dot = 0.f;
    for (int i = 0; i < D; ++i) dot += to_f32(kr[i]) * to_f32(Rg[j * D + i]);
    Zs[idx] = a.sigma * dot;
  }
  __syncthreads();
  const int64_t cap1 = a.dev.ncap[1];
  if (threadIdx.x < R) {
    const int j = threadIdx.x;
    float mx = -INFINITY, sum = 0.f, A = 0.f;
    for (int t = 0; t < nt; ++t) mx = fmaxf(mx, Zs[t * R + j]);
    for (int t = 0; t < nt; ++t) sum += expf(Zs[t * R + j] - mx);
    const float lse = mx + logf(sum);
    for (int t = 0; t < nt; ++t) A += expf(Zs[t * R + j] - lse) * Zs[t * R + j];
    Lj[j] = lse;
    const int64_t gi = ((int64_t)kv * cap1 + n1) * R + j;
    a.dev.c[1][gi] = lse - A;
    a.dev.lse[1][gi] = lse;
  }
  __syncthreads();
  if (a.dev.w1) {
    for (int idx = threadIdx.x; idx < R * a.b; idx += NT) {
      const int j = idx / a.b, k = idx % a.b;
      a.dev.w1[((int64_t)kv * cap1 + n1) * R * a.b + idx] = k < nt ? expf(Zs[k * R + j] - Lj[j]) : 0.f;
    }
  }
  for (int it = threadIdx.x; it < R * (D / 4); it += NT) {
    const int j = it / (D / 4), dc = it % (D / 4);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int t = 0; t < nt; ++t) {
      const TIn* kr = (tb + t == n) ? kn : Kc + (tb + t) * D;
      const float w = expf(Zs[t * R + j] - Lj[j]);
      const float4 k4 = ld4_f32(kr + dc * 4);
      acc.x += w * k4.x; acc.y += w * k4.y; acc.z += w * k4.z; acc.w += w * k4.w;
    }
    *(float4*)(a.dev.s[1] + (((int64_t)kv * cap1 + n1) * R + j) * D + dc * 4) = acc;
  }
  // levels 2..L: one parent each
  int64_t span = a.b;
  for (int v = 2; v <= a.levels; ++v) {
    __threadfence();
    __syncthreads();
    const int64_t nchild = (n + 1 + span - 1) / span;   // nodes at level v-1 after the append
    span *= a.b;
    const int64_t pv = n / span;
    parent_nodes<D, R>(a.dev, v, kv, a.b, pv, 1, nchild, Lp, Wp);
  }
}

// ---------------------------------------------------------------- host launchers
template <typename TIn, int D, int R>
static hipError_t launch_build_d(const BuildArgs& a, int64_t ntiles, int hkv, int T, hipStream_t st) {
  dim3 grid((unsigned)ntiles, (unsigned)hkv);
  if (T == 128) {
    hipLaunchKernelGGL((build_tile_kernel<TIn, D, R, 128>), grid, dim3(256), 0, st, a);
  } else {
    // 256-token tiles (blocks of more than 128 keys) only where the tile fits in LDS
    if constexpr (sizeof(TIn) * 256 * D + 16 * 256 * R <= 160 * 1024)
      hipLaunchKernelGGL((build_tile_kernel<TIn, D, R, 256>), grid, dim3(256), 0, st, a);
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
    dim3 grid((unsigned)((a.nparent + PPB - 1) / PPB), (unsigned)hkv);                     \
    hipLaunchKernelGGL((build_parent_kernel<DD, RR>), grid, dim3(256), 0, st, a);         \
    return hipGetLastError();                                                             \
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
    hipLaunchKernelGGL((append_kernel<TIn, DD, RR>), dim3(hkv), dim3(256), 0, st, a);      \
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
