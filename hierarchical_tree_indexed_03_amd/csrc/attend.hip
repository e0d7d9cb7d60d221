// Attention over the routed keys (and the dense baseline).
//
// Blog "Zyphra Hierarchical Attention", section "Routing through the tree": once the
// search reaches the raw KV entries, ordinary attention runs over the selected subset.
// The level-1 top-p selects blocks; every existing token of a kept block is attended,
// and token 0 is always kept as the attention sink (news summary "Zyphra releases the
// ZHA sparse attention method", section "How does top-p routing pick tokens?").
//
// GPU organisation: split-K flash-decode.  A workgroup owns one KV head and a contiguous
// slice of its gather list (the kept level-1 blocks of the group's union, each with the
// mask of heads that kept it), or of all tokens for the dense baseline.  Each wave takes
// 16 tokens at a time: QK^T for the whole GQA group is one MFMA chain (heads on rows,
// tokens on columns; each lane reads a contiguous quarter of one key row), scores of heads
// that did not keep the token's block are masked, online softmax runs per head, and P.V
// accumulates in fp32 with each lane owning D/64 output dims of every head.  The four
// waves merge in LDS and the workgroup writes one (max, sum, o) partial per head; a
// combine kernel merges the splits and adds the sink.
#include "common.hpp"
#include "kernels.hpp"

namespace zha {

template <typename TIn, int D>
struct QkOps;

template <int D>
struct QkOps<bf16_t, D> {
  static constexpr int NK = D / 32;
  bf16x8 qa[NK];
  __device__ void load_q(const bf16_t* q, int g, int lane) {
    const int row = lane & 15, kg = lane >> 4;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (row < g) v = *(const uint4*)(q + row * D + kg * (D / 4) + kk * 8);
      qa[kk] = __builtin_bit_cast(bf16x8, v);
    }
  }
  __device__ f32x4 scores(const bf16_t* krow, bool valid, int lane) const {
    const int kg = lane >> 4;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (valid) v = *(const uint4*)(krow + kg * (D / 4) + kk * 8);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[kk], __builtin_bit_cast(bf16x8, v), acc, 0, 0, 0);
    }
    return acc;
  }
};

template <int D>
struct QkOps<float, D> {
  float qa[D / 4];
  __device__ void load_q(const float* q, int g, int lane) {
    const int row = lane & 15, kg = lane >> 4;
#pragma unroll
    for (int kk = 0; kk < D / 4; ++kk) qa[kk] = row < g ? q[row * D + kk * 4 + kg] : 0.f;
  }
  __device__ f32x4 scores(const float* krow, bool valid, int lane) const {
    const int kg = lane >> 4;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < D / 4; ++kk) {
      const float kvv = valid ? krow[kk * 4 + kg] : 0.f;
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[kk], kvv, acc, 0, 0, 0);
    }
    return acc;
  }
};

template <int DPL>
__device__ __forceinline__ void load_v(const float* p, float (&v)[DPL]) {
#pragma unroll
  for (int i = 0; i < DPL; ++i) v[i] = p[i];
}
template <int DPL>
__device__ __forceinline__ void load_v(const bf16_t* p, float (&v)[DPL]) {
  if constexpr (DPL == 2) {
    const uint32_t w = *(const uint32_t*)p;
    v[0] = bf16_bits_to_f32(w & 0xffffu);
    v[1] = bf16_bits_to_f32(w >> 16);
  } else {
#pragma unroll
    for (int i = 0; i < DPL; ++i) v[i] = to_f32(p[i]);
  }
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <typename TIn, int D, bool DENSE>
__global__ __launch_bounds__(256) void attend_kernel(AttnArgs a) {
  constexpr int DPL = D / 64;
  __shared__ float Pl[4][16][16];       // [wave][token][head]
  __shared__ float Al[4][16];           // [wave][head] rescale factors
  __shared__ int64_t Tl[4][16];         // [wave][token] token index or -1
  __shared__ float Ml[4][GMAX], Ll[4][GMAX];
  __shared__ float Ol[4][GMAX][D];

  const int kv = blockIdx.y, split = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, kg = lane >> 4;
  const int g = a.g;
  const TIn* Kb = (const TIn*)a.K + (int64_t)kv * a.cap * D;
  const TIn* Vb = (const TIn*)a.V + (int64_t)kv * a.cap * D;
  const TIn* qg = (const TIn*)a.q + (int64_t)kv * g * D;

  int64_t F;
  const int32_t* gnode = nullptr;
  const uint32_t* gmask = nullptr;
  if constexpr (DENSE) {
    F = a.N;
  } else {
    const int64_t cap0 = a.dev.ncap[0];
    F = (int64_t)a.dev.cnt[kv] * a.b;   // level-0 row of the counts: gather list size
    gnode = a.dev.node[0] + kv * cap0;
    gmask = a.dev.mask[0] + kv * cap0;
  }
  int64_t chunk = (F + a.splits - 1) / a.splits;
  chunk = (chunk + 63) / 64 * 64;
  const int64_t fb = (int64_t)split * chunk;
  const int64_t fe = min(fb + chunk, F);

  QkOps<TIn, D> qk;
  qk.load_q(qg, g, lane);

  float m[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) { m[e] = -INFINITY; l[e] = 0.f; }
  float o[GMAX][DPL];
#pragma unroll
  for (int h = 0; h < GMAX; ++h)
#pragma unroll
    for (int i = 0; i < DPL; ++i) o[h][i] = 0.f;

  for (int64_t f0 = fb + wave * 16; f0 < fe; f0 += 64) {
    // token of this lane's column
    const int64_t f = f0 + col;
    bool valid = f < fe;
    int64_t tok = 0;
    uint32_t mk = 0xffffffffu;
    if (valid) {
      if constexpr (DENSE) {
        tok = f;
      } else {
        const int64_t e = f / a.b;
        tok = (int64_t)gnode[e] * a.b + (f - e * a.b);
        mk = gmask[e];
        valid = tok < a.N;
      }
    }
    const f32x4 acc = qk.scores(Kb + tok * D, valid, lane);
    float s[4];
    float rmax[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int h = kg * 4 + e;
      const bool use = valid && h < g && ((mk >> h) & 1u);
      s[e] = use ? a.sigma * acc[e] : -INFINITY;
      rmax[e] = s[e];
    }
#pragma unroll
    for (int off = 1; off < 16; off <<= 1)
#pragma unroll
      for (int e = 0; e < 4; ++e) rmax[e] = fmaxf(rmax[e], __shfl_xor(rmax[e], off));
    float p[4], rsum[4], alpha[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float mn = fmaxf(m[e], rmax[e]);
      alpha[e] = (mn == -INFINITY) ? 1.f : expf(m[e] - mn);
      p[e] = (mn == -INFINITY) ? 0.f : expf(s[e] - mn);
      rsum[e] = p[e];
      m[e] = mn;
    }
#pragma unroll
    for (int off = 1; off < 16; off <<= 1)
#pragma unroll
      for (int e = 0; e < 4; ++e) rsum[e] += __shfl_xor(rsum[e], off);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      l[e] = l[e] * alpha[e] + rsum[e];
      Pl[wave][col][kg * 4 + e] = p[e];
      if (col == 0) Al[wave][kg * 4 + e] = alpha[e];
    }
    if (kg == 0) Tl[wave][col] = valid ? tok : -1;
    wave_sync_lds();
    // P.V: this lane owns dims [lane*DPL, lane*DPL + DPL) of every head.
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
      const float al = Al[wave][h];
#pragma unroll
      for (int i = 0; i < DPL; ++i) o[h][i] *= al;
    }
    for (int t = 0; t < 16; ++t) {
      const int64_t tk = Tl[wave][t];
      if (tk < 0) continue;
      float v[DPL];
      load_v<DPL>(Vb + tk * D + lane * DPL, v);
      const float4 p0 = *(const float4*)&Pl[wave][t][0];
      const float4 p1 = *(const float4*)&Pl[wave][t][4];
      const float ph[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
      for (int h = 0; h < GMAX; ++h)
#pragma unroll
        for (int i = 0; i < DPL; ++i) o[h][i] += ph[h] * v[i];
    }
    wave_sync_lds();
  }
  // merge the four waves
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int h = kg * 4 + e;
    if (col == 0 && h < GMAX) { Ml[wave][h] = m[e]; Ll[wave][h] = l[e]; }
  }
#pragma unroll
  for (int h = 0; h < GMAX; ++h)
#pragma unroll
    for (int i = 0; i < DPL; ++i) Ol[wave][h][lane * DPL + i] = o[h][i];
  __syncthreads();
  for (int idx = threadIdx.x; idx < g * D; idx += 256) {
    const int h = idx / D, d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, Ml[w][h]);
    float L = 0.f, O = 0.f;
    if (M > -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float sc = expf(Ml[w][h] - M);
        L += Ll[w][h] * sc;
        O += Ol[w][h][d] * sc;
      }
    }
    float* pp = a.dev.apart + ((int64_t)(kv * g + h) * MAX_SPLITS + split) * (D + 2);
    if (d == 0) { pp[0] = M; pp[1] = L; }
    pp[2 + d] = O;
  }
}

template <typename TIn, int D, bool DENSE>
__global__ __launch_bounds__(256) void combine_kernel(AttnArgs a, int32_t* stats, int levels) {
  __shared__ float red[256];
  __shared__ float Ms, Ls_, S0;
  const int hq = blockIdx.x, kv = hq / a.g, gi = hq % a.g;
  const float* base = a.dev.apart + (int64_t)hq * MAX_SPLITS * (D + 2);
  const int S = a.splits;
  float mloc = -INFINITY;
  for (int s = threadIdx.x; s < S; s += 256) mloc = fmaxf(mloc, base[(int64_t)s * (D + 2)]);
  red[threadIdx.x] = mloc;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (threadIdx.x < off) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + off]);
    __syncthreads();
  }
  if (threadIdx.x == 0) Ms = red[0];
  __syncthreads();
  const float M = Ms;
  float lloc = 0.f;
  if (M > -INFINITY)
    for (int s = threadIdx.x; s < S; s += 256) {
      const float* pp = base + (int64_t)s * (D + 2);
      lloc += pp[1] * expf(pp[0] - M);
    }
  red[threadIdx.x] = lloc;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) Ls_ = red[0];
  __syncthreads();
  // sink: token 0 if this head did not keep block 0
  bool add_sink = false;
  if constexpr (!DENSE) {
    if (a.keep_sink) {
      const int64_t cap0 = a.dev.ncap[0];
      const bool kept0 = a.dev.cnt[kv] > 0 && a.dev.node[0][kv * cap0] == 0 &&
                         ((a.dev.mask[0][kv * cap0] >> gi) & 1u);
      add_sink = !kept0;
    }
  }
  const TIn* K0 = (const TIn*)a.K + (int64_t)kv * a.cap * D;
  const TIn* V0 = (const TIn*)a.V + (int64_t)kv * a.cap * D;
  if (add_sink) {
    const TIn* qh = (const TIn*)a.q + (int64_t)hq * D;
    float part = 0.f;
    for (int d = threadIdx.x; d < D; d += 256) part += to_f32(qh[d]) * to_f32(K0[d]);
    red[threadIdx.x] = part;
    __syncthreads();
    for (int off = 128; off > 0; off >>= 1) {
      if (threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
      __syncthreads();
    }
    if (threadIdx.x == 0) S0 = a.sigma * red[0];
    __syncthreads();
  }
  for (int d = threadIdx.x; d < D; d += 256) {
    float O = 0.f;
    if (M > -INFINITY)
      for (int s = 0; s < S; ++s) {
        const float* pp = base + (int64_t)s * (D + 2);
        O += pp[2 + d] * expf(pp[0] - M);
      }
    float L = Ls_, Mx = M;
    if (add_sink) {
      const float s0 = S0;
      const float mn = fmaxf(Mx, s0);
      const float sa = (Mx == -INFINITY) ? 0.f : expf(Mx - mn);
      const float sb = expf(s0 - mn);
      O = O * sa + to_f32(V0[d]) * sb;
      L = L * sa + sb;
    }
    a.out[(int64_t)hq * D + d] = L > 0.f ? O / L : 0.f;
  }
  if (stats && hq == 0) {
    for (int i = threadIdx.x; i < (levels + 1) * a.hkv; i += 256) {
      const int row = i / a.hkv, k = i % a.hkv;
      const int lvl = row < levels ? levels - row : 0;
      stats[i] = a.dev.cnt[lvl * a.hkv + k];
    }
  }
}

template <typename TIn, int D, bool DENSE>
static hipError_t launch_attend_t(const AttnArgs& a, int32_t* stats, int levels, hipStream_t st) {
  hipLaunchKernelGGL((attend_kernel<TIn, D, DENSE>), dim3((unsigned)a.splits, (unsigned)a.hkv), dim3(256), 0, st, a);
  hipLaunchKernelGGL((combine_kernel<TIn, D, DENSE>), dim3((unsigned)a.hq), dim3(256), 0, st, a, stats, levels);
  return hipGetLastError();
}

hipError_t launch_attend_full(const AttnArgs& a, bool bf16, int D, bool dense, int32_t* stats, int levels,
                              hipStream_t st) {
#define ZHA_CASE(T, DD, DN) \
  if (D == DD && dense == DN) return launch_attend_t<T, DD, DN>(a, stats, levels, st);
  if (bf16) {
    ZHA_CASE(bf16_t, 64, false) ZHA_CASE(bf16_t, 64, true) ZHA_CASE(bf16_t, 128, false) ZHA_CASE(bf16_t, 128, true)
  } else {
    ZHA_CASE(float, 64, false) ZHA_CASE(float, 64, true) ZHA_CASE(float, 128, false) ZHA_CASE(float, 128, true)
  }
#undef ZHA_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_attend(const AttnArgs& a, bool bf16, int D, bool dense, hipStream_t st) {
  return launch_attend_full(a, bf16, D, dense, nullptr, 0, st);
}

}  // namespace zha
