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
// 32 tokens at a time (all of the tile's K and V loads issued together; other waves of
// the SIMD cover the latency).  S^T = K.Q^T for the whole GQA group is an MFMA
// chain (tokens on rows, heads on columns; each lane reads a contiguous quarter of one key
// row), scores of heads that did not keep the token's block are masked, online softmax
// runs per head, and P.V accumulates in fp32 with each lane owning a 4-element slice of
// the V rows of a subset of the tile's tokens.  The four waves merge in LDS and the
// workgroup writes one (max, sum, o) partial per head; a combine kernel merges the splits
// and adds the sink.
#include "common.hpp"
#include "kernels.hpp"
#include "qk_tile.hpp"
#include "route_util.hpp"

namespace zha {

// V-row slices owned by one lane in P.V: 8 bytes (4 elements) of bf16, 16 bytes of fp32.
template <typename TIn> struct Vec;
template <> struct Vec<bf16_t> {
  static constexpr int N = 4;
  typedef uint2 T;
  __device__ static void to_f32(const uint2& v, float* o) {
    o[0] = bf16_bits_to_f32(v.x & 0xffffu); o[1] = bf16_bits_to_f32(v.x >> 16);
    o[2] = bf16_bits_to_f32(v.y & 0xffffu); o[3] = bf16_bits_to_f32(v.y >> 16);
  }
  __device__ static uint2 zero() { return make_uint2(0, 0); }
};
template <> struct Vec<float> {
  static constexpr int N = 4;
  typedef uint4 T;
  __device__ static void to_f32(const uint4& v, float* o) {
    o[0] = __uint_as_float(v.x); o[1] = __uint_as_float(v.y);
    o[2] = __uint_as_float(v.z); o[3] = __uint_as_float(v.w);
  }
  __device__ static uint4 zero() { return make_uint4(0, 0, 0, 0); }
};


constexpr int ATILE = 32;   // tokens per wave iteration

// Token range of split `split` out of F tokens: chunks are whole multiples of 4 waves x
// one tile; splits beyond the data get an empty range.
__device__ __forceinline__ int64_t split_chunk(int64_t F, int splits) {
  int64_t chunk = (F + splits - 1) / splits;
  const int64_t unit = 4 * ATILE;
  chunk = (chunk + unit - 1) / unit * unit;
  return chunk < unit ? unit : chunk;
}
__device__ __forceinline__ void split_range(int64_t F, int splits, int split, int64_t& fb, int64_t& fe) {
  const int64_t chunk = split_chunk(F, splits);
  fb = (int64_t)split * chunk;
  fe = min(fb + chunk, F);
}

// Routed attention: the KV heads keep different numbers of blocks, so their gather lists
// are cut into chunks of one common length and each head gets as many splits as it has
// chunks (a fixed number of splits per head would leave the launch waiting on the head
// that kept the most).  The chunk is sized for a.splits x Hkv - Hkv splits, so that the
// heads' splits, each head's count rounded up, still fit the a.splits x Hkv workgroups of
// one resident wave (a workgroup past it would run as a tail of one whole chunk), and it
// never gives one head more than MAX_SPLITS.  Every kernel derives it from the level-0
// counts the same way.
__device__ __forceinline__ const int32_t* qcnt(const AttnArgs& a) {
  return a.dev.cnt + (int64_t)blockIdx.y * a.c_stride;   // this launch row's query
}
__device__ __forceinline__ int64_t routed_chunk(const AttnArgs& a) {
  int64_t F = 0, Fmax = 0;
  const int32_t* cnt = qcnt(a);
  for (int k = 0; k < a.hkv; ++k) {
    const int64_t f = (int64_t)cnt[k] * a.b;
    F += f;
    Fmax = f > Fmax ? f : Fmax;
  }
  const int nsp = a.splits * a.hkv - a.hkv;
  const int64_t c1 = split_chunk(F, nsp > 1 ? nsp : 1), c2 = split_chunk(Fmax, MAX_SPLITS);
  return c1 > c2 ? c1 : c2;
}
__device__ __forceinline__ int routed_splits(const AttnArgs& a, int kv, int64_t chunk) {
  const int64_t f = (int64_t)qcnt(a)[kv] * a.b;
  return (int)((f + chunk - 1) / chunk);
}

// The workgroup's KV head, split and token range [fb, fe) of its gather list (or of all N
// tokens for dense attention: grid (splits, Hkv)); false when it has no tokens.  Routed: a
// one-dimensional grid of a.splits x Hkv workgroups over the heads' splits in order.
template <bool DENSE>
__device__ __forceinline__ bool attn_work(const AttnArgs& a, int& kv, int& split, int64_t& fb, int64_t& fe) {
  if constexpr (DENSE) {
    kv = blockIdx.y;
    split = blockIdx.x;
    split_range(a.N, a.splits, split, fb, fe);
    return fb < fe;
  } else {
    const int64_t ch = routed_chunk(a);
    int x = blockIdx.x;
    for (int k = 0; k < a.hkv; ++k) {
      const int sk = routed_splits(a, k, ch);
      if (x < sk) {
        kv = k;
        split = x;
        ZHA_CHECK(a.dev, x < MAX_SPLITS, CHK_SPLITS);
        fb = (int64_t)x * ch;
        fe = min(fb + ch, (int64_t)qcnt(a)[k] * a.b);
        return true;
      }
      x -= sk;
    }
    return false;
  }
}

template <typename TIn, int D, bool DENSE>
__global__ __launch_bounds__(256) void attend_kernel(AttnArgs a) {
  using VT = typename Vec<TIn>::T;
  constexpr int VEC = Vec<TIn>::N;            // elements of a V row per lane
  constexpr int LPRV = D / VEC;               // lanes per V row
  constexpr int TPI = 64 / LPRV;              // V rows per load instruction
  constexpr int NV = ATILE / TPI;             // V loads per lane per tile
  constexpr int NK = Qk<TIn, D>::NL;
  constexpr int NST = ATILE / 16;
  __shared__ int64_t Tl[4][ATILE];
  __shared__ uint32_t Mk[4][ATILE];
  __shared__ __align__(16) float Pl[4][ATILE][GMAX];
  __shared__ float Al[4][GMAX];
  __shared__ float Ml[4][GMAX], Ll[4][GMAX];
  __shared__ float Ol[4][GMAX][D];

  int kv, split;
  int64_t fb, fe;
  if (!attn_work<DENSE>(a, kv, split, fb, fe)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, kg = lane >> 4;
  const int g = a.g;
  const TIn* Kb = (const TIn*)a.K + (int64_t)kv * a.cap * D;
  const TIn* Vb = (const TIn*)a.V + (int64_t)kv * a.cap * D;

  // the gather list: kept level-1 blocks of the group's union (level-0 entries)
  const int32_t* gnode = nullptr;
  const uint32_t* gmask = nullptr;
  if constexpr (!DENSE) {
    const int64_t cap0 = a.dev.ncap[0];
    gnode = a.dev.node[0] + (int64_t)blockIdx.y * a.l_stride + kv * cap0;
    gmask = a.dev.mask[0] + (int64_t)blockIdx.y * a.l_stride + kv * cap0;
  }
  const int64_t qy = DENSE ? 0 : (int64_t)blockIdx.y;   // query of this launch row
  const int64_t qN = a.N + qy * a.n_step;                // tokens the query may attend

  Qk<TIn, D> qk;
  qk.load_q((const TIn*)a.q + qy * a.q_stride + (int64_t)kv * g * D, g, col, kg);

  float m = -INFINITY, l = 0.f;               // softmax state of head `col`
  float o[GMAX][VEC];
#pragma unroll
  for (int h = 0; h < GMAX; ++h)
#pragma unroll
    for (int i = 0; i < VEC; ++i) o[h][i] = 0.f;

  // Token index and head mask of tile position `lane` (the gather-list lookups of the next
  // tile are issued before the current tile's K/V loads, so they are in flight together).
  auto lookup = [&](int64_t f0, int64_t& tok, uint32_t& mk) {
    const int64_t f = f0 + lane;
    tok = -1;
    mk = 0u;
    if (lane < ATILE && f < fe) {
      if constexpr (DENSE) {
        tok = f;
        mk = 0xffffffffu;
      } else {
        const int64_t e = f / a.b;
        const int64_t t = (int64_t)gnode[e] * a.b + (f - e * a.b);
        ZHA_CHECK(a.dev, gnode[e] >= 0 && (int64_t)gnode[e] * a.b < qN, CHK_TOKEN_RANGE);
        if (t < qN) { tok = t; mk = gmask[e]; }
      }
    }
  };
  int64_t ntok;
  uint32_t nmk;
  lookup(fb + wave * ATILE, ntok, nmk);
  for (int64_t f0 = fb + wave * ATILE; f0 < fe; f0 += 4 * ATILE) {
    if (lane < ATILE) {
      Tl[wave][lane] = ntok;
      Mk[wave][lane] = nmk;
    }
    if (f0 + 4 * ATILE < fe) lookup(f0 + 4 * ATILE, ntok, nmk);
    wave_sync_lds();
    uint4 kf[NST][NK];
    VT vf[NV];
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      const int64_t tk = Tl[wave][st * 16 + col];
      if (tk >= 0) Qk<TIn, D>::load_k(Kb + tk * D, kg, kf[st]);
      else
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) kf[st][kk] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int64_t tk = Tl[wave][i * TPI + lane / LPRV];
      vf[i] = tk >= 0 ? *(const VT*)(Vb + tk * D + (lane % LPRV) * VEC) : Vec<TIn>::zero();
    }
    float sc[NST][4];
    float rmax = -INFINITY;
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      const f32x4 acc = qk.mma(kf[st]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = st * 16 + kg * 4 + e;
        const bool use = col < g && ((Mk[wave][t] >> col) & 1u);
        sc[st][e] = use ? a.sigma * acc[e] : -INFINITY;
        rmax = fmaxf(rmax, sc[st][e]);
      }
    }
    rmax = fmaxf(rmax, __shfl_xor(rmax, 16));
    rmax = fmaxf(rmax, __shfl_xor(rmax, 32));
    const float mn = fmaxf(m, rmax);
    const float alpha = (mn == -INFINITY) ? 1.f : expf(m - mn);
    float rsum = 0.f;
#pragma unroll
    for (int st = 0; st < NST; ++st)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p = (mn == -INFINITY) ? 0.f : expf(sc[st][e] - mn);
        rsum += p;
        if (col < GMAX) Pl[wave][st * 16 + kg * 4 + e][col] = p;
      }
    rsum += __shfl_xor(rsum, 16);
    rsum += __shfl_xor(rsum, 32);
    l = l * alpha + rsum;
    m = mn;
    if (kg == 0 && col < GMAX) Al[wave][col] = alpha;
    wave_sync_lds();
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
      const float al = Al[wave][h];
#pragma unroll
      for (int i = 0; i < VEC; ++i) o[h][i] *= al;
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int t = i * TPI + lane / LPRV;
      float v[VEC];
      Vec<TIn>::to_f32(vf[i], v);
      const float4 p0 = *(const float4*)&Pl[wave][t][0];
      const float4 p1 = *(const float4*)&Pl[wave][t][4];
      const float ph[GMAX] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
      for (int h = 0; h < GMAX; ++h)
#pragma unroll
        for (int j = 0; j < VEC; ++j) o[h][j] += ph[h] * v[j];
    }
    wave_sync_lds();
  }
  // lanes sharing output dims hold disjoint token subsets: sum them
#pragma unroll
  for (int off = LPRV; off < 64; off <<= 1)
#pragma unroll
    for (int h = 0; h < GMAX; ++h)
#pragma unroll
      for (int j = 0; j < VEC; ++j) o[h][j] += __shfl_xor(o[h][j], off);
  if (kg == 0 && col < GMAX) { Ml[wave][col] = m; Ll[wave][col] = l; }
  if (lane < LPRV)
#pragma unroll
    for (int h = 0; h < GMAX; ++h)
#pragma unroll
      for (int j = 0; j < VEC; ++j) Ol[wave][h][lane * VEC + j] = o[h][j];
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
    float* pp = a.dev.apart + qy * a.p_stride + ((int64_t)(kv * g + h) * a.pstride + split) * (D + 2);
    if (d == 0) { pp[0] = M; pp[1] = L; }
    pp[2 + d] = O;
  }
}

// Dense bf16 flash-decode (the baseline): P.V on MFMA as well.  (The routed path keeps P.V on
// the VALU: its short per-split streams are bound by the gather-list lookups and K/V load
// latency, where the lighter kernel's higher occupancy wins.)  Per 32-token tile the probabilities are the
// A operand ([heads x tokens], each lane already holds its head's 8 tokens, in the same
// token order as the S^T tile); the V tile is written to LDS transposed ([dim][token], row
// stride VS) and read back as the B operand, 16 output dims per MFMA.
constexpr int VS = 36;   // LDS row stride of the transposed V tile (bf16): 8-byte aligned rows,
                         // the two halves of a wave write disjoint banks

template <int D, bool DENSE>
__global__ __launch_bounds__(256) void attend_mfma_kernel(AttnArgs a) {
  constexpr int NK = Qk<bf16_t, D>::NL;
  constexpr int NST = ATILE / 16;             // = 2
  constexpr int NM = D / 16;                  // output dim blocks (MFMAs per tile)
  __shared__ int64_t Tl[4][ATILE];
  __shared__ uint32_t Mk[4][ATILE];
  __shared__ float Al[4][GMAX];
  __shared__ float Ml[4][GMAX], Ll[4][GMAX];
  // transposed V tiles during the loop; the waves' partial outputs after it
  constexpr int VT_BYTES = 4 * D * VS * 2;
  constexpr int OL_BYTES = 4 * GMAX * D * 4;
  __shared__ __align__(16) unsigned char buf[VT_BYTES > OL_BYTES ? VT_BYTES : OL_BYTES];

  int kv, split;
  int64_t fb, fe;
  if (!attn_work<DENSE>(a, kv, split, fb, fe)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, kg = lane >> 4;
  const int g = a.g;
  const bf16_t* Kb = (const bf16_t*)a.K + (int64_t)kv * a.cap * D;
  const bf16_t* Vb = (const bf16_t*)a.V + (int64_t)kv * a.cap * D;
  uint16_t* Vt = (uint16_t*)buf + wave * D * VS;

  const int32_t* gnode = nullptr;
  const uint32_t* gmask = nullptr;
  if constexpr (!DENSE) {
    const int64_t cap0 = a.dev.ncap[0];
    gnode = a.dev.node[0] + (int64_t)blockIdx.y * a.l_stride + kv * cap0;
    gmask = a.dev.mask[0] + (int64_t)blockIdx.y * a.l_stride + kv * cap0;
  }
  const int64_t qy = DENSE ? 0 : (int64_t)blockIdx.y;   // query of this launch row
  const int64_t qN = a.N + qy * a.n_step;                // tokens the query may attend

  Qk<bf16_t, D> qk;
  qk.load_q((const bf16_t*)a.q + qy * a.q_stride + (int64_t)kv * g * D, g, col, kg);

  float m = -INFINITY, l = 0.f;               // softmax state of head `col`
  f32x4 acc[NM];
#pragma unroll
  for (int i = 0; i < NM; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto lookup = [&](int64_t f0, int64_t& tok, uint32_t& mk) {
    const int64_t f = f0 + lane;
    tok = -1;
    mk = 0u;
    if (lane < ATILE && f < fe) {
      if constexpr (DENSE) {
        tok = f;
        mk = 0xffffffffu;
      } else {
        const int64_t e = f / a.b;
        const int64_t t = (int64_t)gnode[e] * a.b + (f - e * a.b);
        ZHA_CHECK(a.dev, gnode[e] >= 0 && (int64_t)gnode[e] * a.b < qN, CHK_TOKEN_RANGE);
        if (t < qN) { tok = t; mk = gmask[e]; }
      }
    }
  };
  int64_t ntok;
  uint32_t nmk;
  lookup(fb + wave * ATILE, ntok, nmk);
  const int vt = lane & 31, vc = lane >> 5;   // V loads: token vt, dims 16i + 8vc .. +7
  for (int64_t f0 = fb + wave * ATILE; f0 < fe; f0 += 4 * ATILE) {
    if (lane < ATILE) {
      Tl[wave][lane] = ntok;
      Mk[wave][lane] = nmk;
    }
    if (f0 + 4 * ATILE < fe) lookup(f0 + 4 * ATILE, ntok, nmk);
    wave_sync_lds();
    uint4 kf[NST][NK];
    uint4 vv[NM];
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      const int64_t tk = Tl[wave][st * 16 + col];
      if (tk >= 0) Qk<bf16_t, D>::load_k(Kb + tk * D, kg, kf[st]);
      else
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) kf[st][kk] = make_uint4(0, 0, 0, 0);
    }
    {
      const int64_t tk = Tl[wave][vt];
#pragma unroll
      for (int i = 0; i < NM; ++i)
        vv[i] = tk >= 0 ? *(const uint4*)(Vb + tk * D + 16 * i + 8 * vc) : make_uint4(0, 0, 0, 0);
    }
    float sc[NST][4];
    float rmax = -INFINITY;
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      const f32x4 s4 = qk.mma(kf[st]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = st * 16 + kg * 4 + e;
        const bool use = col < g && ((Mk[wave][t] >> col) & 1u);
        sc[st][e] = use ? a.sigma * s4[e] : -INFINITY;
        rmax = fmaxf(rmax, sc[st][e]);
      }
    }
    rmax = fmaxf(rmax, __shfl_xor(rmax, 16));
    rmax = fmaxf(rmax, __shfl_xor(rmax, 32));
    const float mn = fmaxf(m, rmax);
    const float alpha = (mn == -INFINITY) ? 1.f : expf(m - mn);
    float rsum = 0.f;
    uint32_t pb[4];                           // P row of head `col`, bf16 pairs, slot order
#pragma unroll
    for (int st = 0; st < NST; ++st)
#pragma unroll
      for (int e = 0; e < 4; e += 2) {
        const float p0 = (mn == -INFINITY) ? 0.f : expf(sc[st][e] - mn);
        const float p1 = (mn == -INFINITY) ? 0.f : expf(sc[st][e + 1] - mn);
        rsum += p0 + p1;
        pb[st * 2 + e / 2] = f2bf16_bits(p0) | (f2bf16_bits(p1) << 16);
      }
    rsum += __shfl_xor(rsum, 16);
    rsum += __shfl_xor(rsum, 32);
    l = l * alpha + rsum;
    m = mn;
    if (kg == 0 && col < GMAX) Al[wave][col] = alpha;
    // the V tile, transposed: Vt[dim][token]
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      const uint32_t w4[4] = {vv[i].x, vv[i].y, vv[i].z, vv[i].w};
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int d = 16 * i + 8 * vc + k;
        Vt[d * VS + vt] = (uint16_t)((w4[k >> 1] >> (16 * (k & 1))) & 0xffffu);
      }
    }
    wave_sync_lds();
    float ah[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) ah[e] = (4 * kg + e < GMAX) ? Al[wave][4 * kg + e] : 1.f;
    const bf16x8 pa = __builtin_bit_cast(bf16x8, make_uint4(pb[0], pb[1], pb[2], pb[3]));
#pragma unroll
    for (int i = 0; i < NM; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][e] *= ah[e];
      const uint16_t* row = Vt + (16 * i + col) * VS;
      const uint2 lo = *(const uint2*)(row + 4 * kg);
      const uint2 hi = *(const uint2*)(row + 16 + 4 * kg);
      const bf16x8 vb = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
      acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb, acc[i], 0, 0, 0);
    }
    wave_sync_lds();
  }
  __syncthreads();
  // the waves' partials: acc[i][e] = head 4kg+e, dim 16i + col
  float* Ol = (float*)buf;                    // [4][GMAX][D]
  if (kg == 0 && col < GMAX) { Ml[wave][col] = m; Ll[wave][col] = l; }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int h = 4 * kg + e;
    if (h < GMAX)
#pragma unroll
      for (int i = 0; i < NM; ++i) Ol[(wave * GMAX + h) * D + 16 * i + col] = acc[i][e];
  }
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
        const float sw = expf(Ml[w][h] - M);
        L += Ll[w][h] * sw;
        O += Ol[(w * GMAX + h) * D + d] * sw;
      }
    }
    float* pp = a.dev.apart + qy * a.p_stride + ((int64_t)(kv * g + h) * a.pstride + split) * (D + 2);
    if (d == 0) { pp[0] = M; pp[1] = L; }
    pp[2 + d] = O;
  }
}

// Dense bf16 flash-decode with the next tile's K and V loaded while the current one is
// processed: the same arithmetic as attend_mfma_kernel<D, true> (QK and P.V on bf16 MFMA, V
// transposed through LDS), with the loads of tile i + 1 issued before tile i's MFMAs.  The
// loads are unconditional (rows past the split's end clamped to its last token and masked
// afterwards), so the compiler keeps them in flight across the iteration.
template <int D>
__global__ __launch_bounds__(256, 2) void attend_dense_kernel(AttnArgs a) {
  constexpr int NK = Qk<bf16_t, D>::NL;
  constexpr int NST = ATILE / 16;             // = 2
  constexpr int NM = D / 16;                  // output dim blocks (MFMAs per tile)
  __shared__ float Al[4][GMAX];
  __shared__ float Ml[4][GMAX], Ll[4][GMAX];
  constexpr int VT_BYTES = 4 * D * VS * 2;
  constexpr int OL_BYTES = 4 * GMAX * D * 4;
  __shared__ __align__(16) unsigned char buf[VT_BYTES > OL_BYTES ? VT_BYTES : OL_BYTES];

  int kv, split;
  int64_t fb, fe;
  if (!attn_work<true>(a, kv, split, fb, fe)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, kg = lane >> 4;
  const int g = a.g;
  const bf16_t* Kb = (const bf16_t*)a.K + (int64_t)kv * a.cap * D;
  const bf16_t* Vb = (const bf16_t*)a.V + (int64_t)kv * a.cap * D;
  uint16_t* Vt = (uint16_t*)buf + wave * D * VS;

  Qk<bf16_t, D> qk;
  qk.load_q((const bf16_t*)a.q + (int64_t)kv * g * D, g, col, kg);

  float m = -INFINITY, l = 0.f;               // softmax state of head `col`
  f32x4 acc[NM];
#pragma unroll
  for (int i = 0; i < NM; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int vt = lane & 31, vc = lane >> 5;   // V loads: token vt, dims 16i + 8vc .. +7
  auto load = [&](int64_t f0, uint4 (&kf)[NST][NK], uint4 (&vv)[NM]) {
#pragma unroll
    for (int st = 0; st < NST; ++st)
      Qk<bf16_t, D>::load_k(Kb + min(f0 + st * 16 + col, fe - 1) * D, kg, kf[st]);
    const int64_t tk = min(f0 + vt, fe - 1);
#pragma unroll
    for (int i = 0; i < NM; ++i) vv[i] = *(const uint4*)(Vb + tk * D + 16 * i + 8 * vc);
  };
  // two register sets take turns (no copies: a copy of a register still being loaded makes
  // the compiler wait for the load, which would drain the prefetch)
  uint4 kfa[NST][NK], vva[NM], kfb[NST][NK], vvb[NM];
  auto step = [&](int64_t f0, const uint4 (&kf)[NST][NK], const uint4 (&vv)[NM], uint4 (&kn)[NST][NK],
                  uint4 (&vn)[NM]) {
    load(f0 + 4 * ATILE, kn, vn);             // clamped: past the end it rereads the last row
    float sc[NST][4];
    float rmax = -INFINITY;
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      const f32x4 s4 = qk.mma(kf[st]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool use = col < g && f0 + st * 16 + kg * 4 + e < fe;
        sc[st][e] = use ? a.sigma * s4[e] : -INFINITY;
        rmax = fmaxf(rmax, sc[st][e]);
      }
    }
    rmax = fmaxf(rmax, __shfl_xor(rmax, 16));
    rmax = fmaxf(rmax, __shfl_xor(rmax, 32));
    const float mn = fmaxf(m, rmax);
    const float alpha = (mn == -INFINITY) ? 1.f : expf(m - mn);
    float rsum = 0.f;
    uint32_t pb[4];                           // P row of head `col`, bf16 pairs, slot order
#pragma unroll
    for (int st = 0; st < NST; ++st)
#pragma unroll
      for (int e = 0; e < 4; e += 2) {
        const float p0 = (mn == -INFINITY) ? 0.f : expf(sc[st][e] - mn);
        const float p1 = (mn == -INFINITY) ? 0.f : expf(sc[st][e + 1] - mn);
        rsum += p0 + p1;
        pb[st * 2 + e / 2] = f2bf16_bits(p0) | (f2bf16_bits(p1) << 16);
      }
    rsum += __shfl_xor(rsum, 16);
    rsum += __shfl_xor(rsum, 32);
    l = l * alpha + rsum;
    m = mn;
    if (kg == 0 && col < GMAX) Al[wave][col] = alpha;
    // the V tile, transposed: Vt[dim][token] (rows past the end are weighted 0)
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      const uint32_t w4[4] = {vv[i].x, vv[i].y, vv[i].z, vv[i].w};
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int d = 16 * i + 8 * vc + k;
        Vt[d * VS + vt] = (uint16_t)((w4[k >> 1] >> (16 * (k & 1))) & 0xffffu);
      }
    }
    wave_sync_lds();
    float ah[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) ah[e] = (4 * kg + e < GMAX) ? Al[wave][4 * kg + e] : 1.f;
    const bf16x8 pa = __builtin_bit_cast(bf16x8, make_uint4(pb[0], pb[1], pb[2], pb[3]));
#pragma unroll
    for (int i = 0; i < NM; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][e] *= ah[e];
      const uint16_t* row = Vt + (16 * i + col) * VS;
      const uint2 lo = *(const uint2*)(row + 4 * kg);
      const uint2 hi = *(const uint2*)(row + 16 + 4 * kg);
      const bf16x8 vb = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
      acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb, acc[i], 0, 0, 0);
    }
    wave_sync_lds();
  };
  load(fb + wave * ATILE, kfa, vva);
  for (int64_t f0 = fb + wave * ATILE; f0 < fe; f0 += 8 * ATILE) {
    step(f0, kfa, vva, kfb, vvb);
    if (f0 + 4 * ATILE >= fe) break;
    step(f0 + 4 * ATILE, kfb, vvb, kfa, vva);
  }
  __syncthreads();
  // the waves' partials: acc[i][e] = head 4kg+e, dim 16i + col
  float* Ol = (float*)buf;                    // [4][GMAX][D]
  if (kg == 0 && col < GMAX) { Ml[wave][col] = m; Ll[wave][col] = l; }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int h = 4 * kg + e;
    if (h < GMAX)
#pragma unroll
      for (int i = 0; i < NM; ++i) Ol[(wave * GMAX + h) * D + 16 * i + col] = acc[i][e];
  }
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
        const float sw = expf(Ml[w][h] - M);
        L += Ll[w][h] * sw;
        O += Ol[(w * GMAX + h) * D + d] * sw;
      }
    }
    float* pp = a.dev.apart + ((int64_t)(kv * g + h) * a.pstride + split) * (D + 2);
    if (d == 0) { pp[0] = M; pp[1] = L; }
    pp[2 + d] = O;
  }
}

template <typename TIn, int D, bool DENSE>
__global__ __launch_bounds__(512) void combine_kernel(AttnArgs a, int32_t* stats, int levels) {
  constexpr int NW = 8;        // waves: split rows are dealt round-robin to the waves
  constexpr int VD = D / 64;   // output dims per lane
  __shared__ float Wl[MAX_SPLITS];
  __shared__ float redm[NW], redl[NW];
  __shared__ float Ored[NW][D];
  __shared__ float S0;
  const int hq = blockIdx.x, kv = hq / a.g, gi = hq % a.g;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t qy = blockIdx.y;              // query of this launch row (0 for a decode)
  const float* base = a.dev.apart + qy * a.p_stride + (int64_t)hq * a.pstride * (D + 2);
  // splits that own tokens (same chunking as the attention kernel)
  int S = 0;
  if constexpr (DENSE) {
    const int64_t F = a.N;
    if (F > 0) {
      const int64_t ch = split_chunk(F, a.splits);
      const int64_t s = (F + ch - 1) / ch;
      S = s < a.splits ? (int)s : a.splits;
    }
  } else {
    S = routed_splits(a, kv, routed_chunk(a));
  }
  // pass 1: max of the partial maxima
  float ms = -INFINITY, ls = 0.f;
  if ((int)threadIdx.x < S) { ms = base[(int64_t)threadIdx.x * (D + 2)]; ls = base[(int64_t)threadIdx.x * (D + 2) + 1]; }
  float mx = ms;
  for (int s = threadIdx.x + 512; s < S; s += 512) mx = fmaxf(mx, base[(int64_t)s * (D + 2)]);
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if (lane == 0) redm[wave] = mx;
  // sink: token 0 when this head did not keep block 0
  bool add_sink = false;
  if constexpr (!DENSE) {
    if (a.keep_sink) {
      const int64_t cap0 = a.dev.ncap[0];
      const int64_t l0 = qy * a.l_stride + kv * cap0;
      const bool kept0 = qcnt(a)[kv] > 0 && a.dev.node[0][l0] == 0 && ((a.dev.mask[0][l0] >> gi) & 1u);
      add_sink = !kept0;
    }
  }
  const TIn* K0 = (const TIn*)a.K + (int64_t)kv * a.cap * D;
  const TIn* V0 = (const TIn*)a.V + (int64_t)kv * a.cap * D;
  if (add_sink && wave == NW - 1) {
    const TIn* qh = (const TIn*)a.q + qy * a.q_stride + (int64_t)hq * D;
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < VD; ++i) part += to_f32(qh[lane * VD + i]) * to_f32(K0[lane * VD + i]);
    for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off);
    if (lane == 0) S0 = a.sigma * part;
  }
  __syncthreads();
  float M = redm[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) M = fmaxf(M, redm[w]);
  // weights and the softmax denominator
  float lsum = 0.f;
  for (int s = threadIdx.x; s < S; s += 512) {
    const float m_s = s == (int)threadIdx.x ? ms : base[(int64_t)s * (D + 2)];
    const float l_s = s == (int)threadIdx.x ? ls : base[(int64_t)s * (D + 2) + 1];
    const float w = (M > -INFINITY && l_s > 0.f) ? expf(m_s - M) : 0.f;
    Wl[s] = w;
    lsum += l_s * w;
  }
  for (int off = 32; off > 0; off >>= 1) lsum += __shfl_xor(lsum, off);
  if (lane == 0) redl[wave] = lsum;
  __syncthreads();
  // pass 2: weighted sum of the split outputs, rows round-robin over the waves
  float O[VD];
#pragma unroll
  for (int i = 0; i < VD; ++i) O[i] = 0.f;
  int s = wave;
  for (; s + 7 * NW < S; s += 8 * NW) {
    float v[8][VD];
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int i = 0; i < VD; ++i) v[u][i] = base[(int64_t)(s + u * NW) * (D + 2) + 2 + lane * VD + i];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float w = Wl[s + u * NW];
#pragma unroll
      for (int i = 0; i < VD; ++i) O[i] += w * v[u][i];
    }
  }
  for (; s < S; s += NW) {
    const float w = Wl[s];
#pragma unroll
    for (int i = 0; i < VD; ++i) O[i] += w * base[(int64_t)s * (D + 2) + 2 + lane * VD + i];
  }
#pragma unroll
  for (int i = 0; i < VD; ++i) Ored[wave][lane * VD + i] = O[i];
  __syncthreads();
  for (int d = threadIdx.x; d < D; d += 512) {
    float Ov = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) Ov += Ored[w][d];
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) L += redl[w];
    if (add_sink) {
      const float s0 = S0;
      const float mn = fmaxf(M, s0);
      const float sa = (M == -INFINITY) ? 0.f : expf(M - mn);
      const float sb = expf(s0 - mn);
      Ov = Ov * sa + to_f32(V0[d]) * sb;
      L = L * sa + sb;
    }
    a.out[qy * a.o_stride + (int64_t)hq * D + d] = L > 0.f ? Ov / L : 0.f;
  }
  if (stats && hq == 0 && qy == 0) {
    for (int i = threadIdx.x; i < (levels + 1) * a.hkv; i += 512) {
      const int row = i / a.hkv, k = i % a.hkv;
      const int lvl = row < levels ? levels - row : 0;
      stats[i] = a.dev.ucnt[lvl * a.hkv + k];
    }
  }
}

// Dense bf16 attention runs P.V on MFMA; routed attention keeps P.V on the VALU (its MFMA
// variant measured slower on every routed workload: lower occupancy, short gathers).
template <typename TIn, int D, bool DENSE>
static hipError_t launch_attend_t(const AttnArgs& a, int32_t* stats, int levels, hipStream_t st) {
  // dense: (splits, Hkv); routed: one dimension over every head's splits (see attn_work)
  const dim3 grid = DENSE ? dim3((unsigned)a.splits, (unsigned)a.hkv) : dim3((unsigned)(a.splits * a.hkv));
  if constexpr (sizeof(TIn) == 2 && DENSE)
    hipLaunchKernelGGL((attend_dense_kernel<D>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((attend_kernel<TIn, D, DENSE>), grid, dim3(256), 0, st, a);
  hipLaunchKernelGGL((combine_kernel<TIn, D, DENSE>), dim3((unsigned)a.hq), dim3(512), 0, st, a, stats, levels);
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

template <typename TIn, int D, bool DENSE>
static int resident_splits_t(int hkv) {
  static const int per_cu = [] {
    if constexpr (sizeof(TIn) == 2 && DENSE) return resident_per_cu(attend_dense_kernel<D>, 256);
    else return resident_per_cu(attend_kernel<TIn, D, DENSE>, 256);
  }();
  const int s = per_cu * device_cus() / hkv;
  return s > MAX_SPLITS ? MAX_SPLITS : (s < 1 ? 1 : s);
}

int attend_resident_splits(bool bf16, int D, bool dense, int hkv) {
#define ZHA_CASE(T, DD, DN) \
  if (D == DD && dense == DN) return resident_splits_t<T, DD, DN>(hkv);
  if (bf16) {
    ZHA_CASE(bf16_t, 64, false) ZHA_CASE(bf16_t, 64, true) ZHA_CASE(bf16_t, 128, false) ZHA_CASE(bf16_t, 128, true)
  } else {
    ZHA_CASE(float, 64, false) ZHA_CASE(float, 64, true) ZHA_CASE(float, 128, false) ZHA_CASE(float, 128, true)
  }
#undef ZHA_CASE
  return 1;
}

template <typename TIn, int D>
static hipError_t launch_attend_batch_t(const AttnArgs& a, int nq, hipStream_t st) {
  hipLaunchKernelGGL((attend_kernel<TIn, D, false>), dim3((unsigned)(a.splits * a.hkv), (unsigned)nq), dim3(256), 0, st, a);
  hipLaunchKernelGGL((combine_kernel<TIn, D, false>), dim3((unsigned)a.hq, (unsigned)nq), dim3(512), 0, st, a,
                     (int32_t*)nullptr, 0);
  return hipGetLastError();
}

hipError_t launch_attend_batch(const AttnArgs& a, bool bf16, int D, int nq, hipStream_t st) {
  if (bf16) {
    if (D == 64) return launch_attend_batch_t<bf16_t, 64>(a, nq, st);
    if (D == 128) return launch_attend_batch_t<bf16_t, 128>(a, nq, st);
  } else {
    if (D == 64) return launch_attend_batch_t<float, 64>(a, nq, st);
    if (D == 128) return launch_attend_batch_t<float, 128>(a, nq, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attend(const AttnArgs& a, bool bf16, int D, bool dense, hipStream_t st) {
  return launch_attend_full(a, bf16, D, dense, nullptr, 0, st);
}

}  // namespace zha
