// Batched causal prefill: the queries of mb consecutive positions routed together.
//
// The method's attention cost is subquadratic in the context as a whole, prefill included
// (paper abstract, "Subquadratic Attention with a Hierarchical Tree-Structured Indexer";
// blog "Zyphra Hierarchical Attention", section "How is this subquadratic"): query i of a
// prompt chunk routes over the tree of the tokens up to and including its own, exactly as a
// decode step would (blog, "Routing through the tree").  Its tree differs from the tree over
// the whole chunk only in the rightmost node of each level, which covers part of the chunk:
// every node to its left is complete in both, and the nodes to its right do not exist yet.
//
// So, per sub-batch of mb queries (after the chunk's tokens are in the tree):
//   prefix   one workgroup per (query, KV head) builds that query's own rightmost node of
//            every level: level 1 from the keys up to its position, each level above from
//            the complete children to its left (read from the tree) and its own node one
//            level down (the build's arithmetic: logsumexp of the children's log masses,
//            their softmax-weighted mean s and A = sigma r.s, c = LSE - A);
//   score    every node of every level of the tree, for all mb * g (query, head) pairs of
//            a KV head: each 16-row plane tile is read once and multiplied on fp32 MFMA with
//            the queries 16 pairs at a time;
//   tail     each pair's scores right of its own rightmost node become -inf (no node) and
//            the rightmost node's score comes from the pair's own version of it;
//   select   one workgroup per pair walks the levels from the top: the frontier is the
//            children of the nodes it kept one level up, the same fixed-point top-p decision
//            as a decode (coarse and fine mass histograms, exact rank order on ties), scores
//            read from global memory, kept bitmaps written to global memory;
//   gather   per (query, KV head), the kept level-1 blocks of the query's heads with their
//            head masks, in block order: the query's gather list;
// then the routed attention runs for all mb queries in one launch (grid.y = query).
#include "common.hpp"
#include "kernels.hpp"
#include "route_util.hpp"

namespace zha {

// ---------------------------------------------------------------- prefix nodes
constexpr int PX_BMAX = 256;   // largest block

template <typename TIn, int D, int R>
__global__ __launch_bounds__(256) void prefill_prefix_kernel(PrefillArgs a) {
  __shared__ float Wt[R * PX_BMAX];   // per plane: token / child weights of the node being built
  __shared__ float LS[R], AS[R];
  const int i = blockIdx.x, kv = blockIdx.y, tid = threadIdx.x;
  const int b = a.b, L = a.levels;
  const int lb = __ffs(b) - 1;
  const int64_t pos = a.N0 + i;        // the query's own token: its tree holds [0, pos]
  const TIn* Kc = (const TIn*)a.K + (int64_t)kv * a.cap * D;
  const TIn* Rg = (const TIn*)a.refs + (int64_t)kv * R * D;
  float* Xq = a.X + ((int64_t)kv * a.mbmax + i) * (a.levels + 1) * R * (D + 2);
  // ---- level 1: the keys [t0, pos] of the query's block
  {
    const int64_t t0 = (pos >> lb) << lb;
    const int nt = (int)(pos - t0 + 1);
    for (int idx = tid; idx < R * nt; idx += 256) {
      const int j = idx / nt, t = idx % nt;
      float acc = 0.f;
      for (int d = 0; d < D; ++d) acc += to_f32(Rg[j * D + d]) * to_f32(Kc[(t0 + t) * D + d]);
      Wt[j * PX_BMAX + t] = a.sigma * acc;                    // logit z
    }
    __syncthreads();
    if (tid < R) {
      const int j = tid;
      float mx = -INFINITY;
      for (int t = 0; t < nt; ++t) mx = fmaxf(mx, Wt[j * PX_BMAX + t]);
      float sum = 0.f;
      for (int t = 0; t < nt; ++t) sum += expf(Wt[j * PX_BMAX + t] - mx);
      const float lse = mx + logf(sum);
      float A = 0.f;
      for (int t = 0; t < nt; ++t) {
        const float z = Wt[j * PX_BMAX + t];
        const float w = expf(z - lse);
        A += w * z;
        Wt[j * PX_BMAX + t] = w;                              // weight
      }
      LS[j] = lse;
      AS[j] = A;
    }
    __syncthreads();
    float* X1 = Xq + 1 * R * (D + 2);
    for (int idx = tid; idx < R * D; idx += 256) {
      const int j = idx / D, d = idx % D;
      float s = 0.f;
      for (int t = 0; t < nt; ++t) s += Wt[j * PX_BMAX + t] * to_f32(Kc[(t0 + t) * D + d]);
      X1[j * (D + 2) + d] = s;
    }
    if (tid < R) {
      X1[tid * (D + 2) + D] = LS[tid] - AS[tid];
      X1[tid * (D + 2) + D + 1] = LS[tid];
    }
    __syncthreads();
  }
  // ---- levels 2..L: complete children from the tree, the last child the query's own node
  for (int lv = 2; lv <= L; ++lv) {
    const int64_t pc = pos >> (lb * (lv - 1));                // the query's node one level down
    const int64_t c0 = (pos >> (lb * lv)) << lb;              // first child of its node here
    const int nc = (int)(pc - c0);                            // complete children
    const int64_t ccap = a.dev.ncap[lv - 1];
    const float* lse_c = a.dev.lse[lv - 1] + ((int64_t)kv * ccap + c0) * R;
    const float* c_c = a.dev.c[lv - 1] + ((int64_t)kv * ccap + c0) * R;
    const float* s_c = a.dev.s[lv - 1] + ((int64_t)kv * ccap + c0) * R * D;
    const float* Xp = Xq + (lv - 1) * R * (D + 2);
    float* Xl = Xq + lv * R * (D + 2);
    if (tid < R) {
      const int j = tid;
      const float lx = Xp[j * (D + 2) + D + 1];
      float mx = lx;
      for (int c = 0; c < nc; ++c) mx = fmaxf(mx, lse_c[c * R + j]);
      float sum = expf(lx - mx);
      for (int c = 0; c < nc; ++c) sum += expf(lse_c[c * R + j] - mx);
      const float lse = mx + logf(sum);
      float A = 0.f;
      for (int c = 0; c < nc; ++c) {
        const float lc = lse_c[c * R + j];
        const float w = expf(lc - lse);
        Wt[j * PX_BMAX + c] = w;
        A += w * (lc - c_c[c * R + j]);
      }
      const float wx = expf(lx - lse);
      Wt[j * PX_BMAX + nc] = wx;
      A += wx * (lx - Xp[j * (D + 2) + D]);
      LS[j] = lse;
      AS[j] = A;
    }
    __syncthreads();
    for (int idx = tid; idx < R * D; idx += 256) {
      const int j = idx / D, d = idx % D;
      float s = Wt[j * PX_BMAX + nc] * Xp[j * (D + 2) + d];
      for (int c = 0; c < nc; ++c) s += Wt[j * PX_BMAX + c] * s_c[((int64_t)c * R + j) * D + d];
      Xl[j * (D + 2) + d] = s;
    }
    if (tid < R) {
      Xl[tid * (D + 2) + D] = LS[tid] - AS[tid];
      Xl[tid * (D + 2) + D + 1] = LS[tid];
    }
    __syncthreads();
  }
}

// sigma * q in fp32, pair order p = i * g + gi within each KV head
template <typename TIn, int D>
__global__ __launch_bounds__(256) void prefill_qprep_kernel(PrefillArgs a) {
  const TIn* q = (const TIn*)a.q;
  const int64_t tot = (int64_t)a.mb * a.hq * D;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < tot; idx += (int64_t)gridDim.x * 256) {
    const int64_t i = idx / ((int64_t)a.hq * D);
    const int64_t rem = idx % ((int64_t)a.hq * D);
    const int h = (int)(rem / D), d = (int)(rem % D);
    const int kv = h / a.g, gi = h % a.g;
    a.Qf[((int64_t)kv * a.P + i * a.g + gi) * D + d] = a.sigma * to_f32(q[idx]);
  }
}

// ---------------------------------------------------------------- batched scoring
// The fp32 plane scorer's tile (16 plane rows = 16/R nodes, read whole and transposed
// through LDS into the MFMA layout) against every block of 16 pairs in turn: the tile is
// read from HBM once, the pairs' queries (8 KB per block) come from L2, the next block's
// queries are loaded during the current block's MFMAs.  Grid: (tiles, Hkv, levels), level 1
// (the largest) first.
template <int D, int R>
__global__ __launch_bounds__(256) void prefill_score_kernel(PrefillArgs a) {
  constexpr int NPT = 16 / R;
  constexpr int NI = D / 16;
  constexpr int LPR = D / 4;
  constexpr int RPI = 64 / LPR;
  constexpr int NLD = 16 / RPI;
  constexpr int RS = D + 4;
  __shared__ __align__(16) float stg[4][16 * RS];
  const int kv = blockIdx.y, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, kg = lane >> 4;
  const int slot = col / R, plane = col % R;
  const int lrow = lane / LPR, lcol = (lane % LPR) * 4;
  const int lv = 1 + (int)blockIdx.z;
  const int64_t n = a.nl[lv];
  const int64_t cap = a.dev.ncap[lv];
  const float* S = a.dev.s[lv] + (int64_t)kv * cap * R * D;
  const float* C = a.dev.c[lv] + (int64_t)kv * cap * R;
  const int64_t sst = a.sstride[lv];
  float* out = a.S + a.soff[lv] + (int64_t)kv * a.P * sst;
  const float* Qf = a.Qf + (int64_t)kv * a.P * D;
  float* W = stg[wave];
  const int P = a.P, npb = (P + 15) / 16;

  auto load_q = [&](int pb, float (&qa)[NI][4]) {
    const int p = pb * 16 + col;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (p < P) x = *(const float4*)(Qf + (int64_t)p * D + 16 * i + 4 * kg);
      qa[i][0] = x.x; qa[i][1] = x.y; qa[i][2] = x.z; qa[i][3] = x.w;
    }
  };
  const int64_t ntiles = (n + NPT - 1) / NPT;
  const int64_t tstride = (int64_t)gridDim.x * 4;
  int32_t rnid;
  float rcj;
  uint4 ld[NLD];
  auto fetch = [&](int64_t t) {
    const int64_t e = t * NPT + slot;
    rnid = (t < ntiles && e < n) ? (int32_t)e : -1;
    rcj = rnid >= 0 ? C[(int64_t)rnid * R + plane] : -INFINITY;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int r = lrow + RPI * i;
      const int32_t nd = __shfl(rnid, r);
      ld[i] = nd >= 0 ? *(const uint4*)(S + ((int64_t)nd * R + r % R) * D + lcol) : make_uint4(0, 0, 0, 0);
    }
  };
  int64_t t = (int64_t)blockIdx.x * 4 + wave;
  if (t < ntiles) fetch(t);
  for (; t < ntiles; t += tstride) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) *(uint4*)(W + (lrow + RPI * i) * RS + lcol) = ld[i];
    const int32_t nid = rnid;
    const float cj = rcj;
    wave_sync_lds();
    if (t + tstride < ntiles) fetch(t + tstride);
    float4 sb[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) sb[i] = *(const float4*)(W + col * RS + 16 * i + 4 * kg);
    wave_sync_lds();
    float qa[NI][4], qn[NI][4];
    load_q(0, qa);
    for (int pb = 0; pb < npb; ++pb) {
      if (pb + 1 < npb) load_q(pb + 1, qn);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[i][0], sb[i].x, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[i][1], sb[i].y, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[i][2], sb[i].z, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[i][3], sb[i].w, acc, 0, 0, 0);
      }
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = acc[e] + cj;
#pragma unroll
      for (int off = 1; off < R; off <<= 1)
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = fmaxf(v[e], __shfl_xor(v[e], off));
      if (nid >= 0 && plane == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int p = pb * 16 + kg * 4 + e;
          if (p < P) out[(int64_t)p * sst + nid] = v[e];
        }
      }
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int k = 0; k < 4; ++k) qa[i][k] = qn[i][k];
    }
  }
}

// Each pair's tail: nodes right of its own rightmost node do not exist (-inf), the rightmost
// node scores with the pair's own version of it.  Grid (P, Hkv, levels); one wave per
// workgroup computes the R plane values of the own node.
template <int D, int R>
__global__ __launch_bounds__(64) void prefill_tail_kernel(PrefillArgs a) {
  const int p = blockIdx.x, kv = blockIdx.y, lv = 1 + (int)blockIdx.z, lane = threadIdx.x;
  const int i = p / a.g;
  const int lb = __ffs(a.b) - 1;
  const int64_t own = (a.N0 + i) >> (lb * lv);
  const int64_t n = a.nl[lv];
  const int64_t sst = a.sstride[lv];
  float* row = a.S + a.soff[lv] + ((int64_t)kv * a.P + p) * sst;
  const float* q = a.Qf + ((int64_t)kv * a.P + p) * D;
  const float* Xl = a.X + ((int64_t)kv * a.mbmax + i) * (a.levels + 1) * R * (D + 2) + lv * R * (D + 2);
  float best = -INFINITY;
  for (int j = 0; j < R; ++j) {
    float part = 0.f;
    for (int d = lane; d < D; d += 64) part += q[d] * Xl[j * (D + 2) + d];
    for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off);
    best = fmaxf(best, part + Xl[j * (D + 2) + D]);
  }
  if (lane == 0) row[own] = best;
  for (int64_t e = own + 1 + lane; e < n; e += 64) row[e] = -INFINITY;
}

// ---------------------------------------------------------------- per-pair selection
constexpr int PS_THREADS = 512;
constexpr int PS_LIST = 8192;   // frontier nodes held in LDS (more: the level is read from global memory)
constexpr int PS_TIES = 256;    // boundary sub-bin nodes resolved pairwise (more: radix select)

// Kept bitmap words written earlier in the same workgroup (stores and L2 atomics): read at
// agent scope so that no stale vector-cache line is returned.
__device__ __forceinline__ uint32_t ld_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One wave: the first of 512 bins where base + inclusive prefix >= target, and the mass
// before it; the bins' total.
__device__ __forceinline__ void ps_find(const unsigned long long* bins, uint64_t base, uint64_t target, uint32_t& bin,
                                        uint64_t& above, uint64_t& total) {
  const int lane = threadIdx.x & 63;
  uint64_t v[8], loc = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) { v[k] = bins[lane * 8 + k]; loc += v[k]; }
  uint64_t inc = loc;
  for (int off = 1; off < 64; off <<= 1) {
    const uint64_t x = __shfl_up(inc, off);
    if (lane >= off) inc += x;
  }
  total = __shfl(inc, 63);
  uint64_t run = base + inc - loc;
  uint32_t fb = 0xffffffffu;
  uint64_t fa = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (fb == 0xffffffffu && run < target && run + v[k] >= target) { fb = lane * 8 + k; fa = run; }
    run += v[k];
  }
  const uint64_t hit = __ballot(fb != 0xffffffffu);
  const int src = hit ? __ffsll((long long)hit) - 1 : 0;
  bin = __shfl(fb, src);
  above = __shfl(fa, src);
}

// Exclusive prefix of `v` over the workgroup (PS_THREADS threads) and the total.
__device__ __forceinline__ int32_t ps_scan(int32_t v, int32_t* wsum, int32_t& total) {
  constexpr int NW = PS_THREADS / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int32_t inc = v;
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t x = __shfl_up(inc, off);
    if (lane >= off) inc += x;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  int32_t pre = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    pre += w < wave ? wsum[w] : 0;
    tot += wsum[w];
  }
  __syncthreads();
  total = tot;
  return pre + inc - v;
}

// One workgroup per (pair, KV head) walks the levels from the top.  The level's frontier
// (every node at the top, else the children of the nodes kept one level up, in node order)
// is listed in LDS with its scores; a frontier longer than PS_LIST is read from global
// memory on every pass instead.  Nodes outside the pair's tree score -inf and drop out.
__global__ __launch_bounds__(PS_THREADS) void prefill_select_kernel(PrefillArgs a) {
  constexpr int NW = PS_THREADS / 64;
  __shared__ int32_t fl[PS_LIST];
  __shared__ float fs[PS_LIST];
  __shared__ unsigned long long h[NB1];
  __shared__ int32_t tie_e[PS_TIES];
  __shared__ float tie_s[PS_TIES];
  __shared__ uint64_t tie_m[PS_TIES];
  __shared__ float redm[NW];
  __shared__ int32_t wsum[NW];
  __shared__ uint32_t s_b1, s_b2, s_ntie;
  __shared__ uint64_t s_T, s_above1, s_above2, s_prefix, s_rabove;
  static_assert(NB1 == 512 && NB2 == 512, "ps_find scans 512 bins");
  const int p = blockIdx.x, kv = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = a.b, lb = __ffs(b) - 1;
  const int L = a.levels;
  for (int lv = L; lv >= 1; --lv) {
    const int64_t n = a.nl[lv];
    const int64_t nw = (n + 31) >> 5;
    const bool top = lv == L;
    const float* row = a.S + a.soff[lv] + ((int64_t)kv * a.P + p) * a.sstride[lv];
    uint32_t* kb = a.KB + a.koff[lv] + ((int64_t)kv * a.P + p) * a.kstride[lv];
    const uint32_t* kp = top ? nullptr : a.KB + a.koff[lv + 1] + ((int64_t)kv * a.P + p) * a.kstride[lv + 1];
    for (int64_t w = tid; w < nw; w += PS_THREADS) kb[w] = 0u;
    // ---- the frontier
    int64_t nf = 0;
    if (top) {
      nf = n;
      if (n <= PS_LIST)
        for (int k = tid; k < (int)n; k += PS_THREADS) { fl[k] = k; fs[k] = row[k]; }
    } else {
      const int64_t np = a.nl[lv + 1];
      const int64_t nwp = (np + 31) >> 5;
      for (int64_t w0 = 0; w0 < nwp; w0 += PS_THREADS) {
        const int64_t w = w0 + tid;
        const uint32_t word = w < nwp ? ld_agent(kp + w) : 0u;
        int32_t cnt = 0;
        for (uint32_t r = word; r; r &= r - 1u) {
          const int64_t first = (32 * w + __ffs(r) - 1) << lb;
          cnt += (int32_t)min((int64_t)b, n - first);
        }
        int32_t round;
        int64_t off = nf + ps_scan(cnt, wsum, round);
        if (nf + round <= PS_LIST) {
          for (uint32_t r = word; r; r &= r - 1u) {
            const int64_t first = (32 * w + __ffs(r) - 1) << lb;
            const int64_t last = min(first + b, n);
            for (int64_t e = first; e < last; ++e, ++off) { fl[off] = (int32_t)e; fs[off] = row[e]; }
          }
        }
        nf += round;
      }
    }
    const bool list = nf <= PS_LIST;
    const int64_t count = list ? nf : n;
    // (node, score) of entry k; -inf outside the frontier
    auto get = [&](int64_t k, int64_t& e, float& x) {
      if (list) {
        e = fl[k];
        x = fs[k];
      } else {
        e = k;
        bool in = top;
        if (!in) {
          const int64_t pn = k >> lb;
          in = (ld_agent(kp + (pn >> 5)) >> (pn & 31)) & 1u;
        }
        x = in ? row[k] : -INFINITY;
      }
    };
    __syncthreads();
    // ---- max
    float mx = -INFINITY;
    for (int64_t k = tid; k < count; k += PS_THREADS) {
      int64_t e;
      float x;
      get(k, e, x);
      mx = fmaxf(mx, x);
    }
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    if (lane == 0) redm[wave] = mx;
    for (int k = tid; k < NB1; k += PS_THREADS) h[k] = 0ull;
    __syncthreads();
    float M = redm[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, redm[w]);
    if (M == -INFINITY) {   // empty frontier: nothing kept here or below
      __syncthreads();
      continue;
    }
    // ---- coarse histogram of the fixed-point masses
    for (int64_t k = tid; k < count; k += PS_THREADS) {
      int64_t e;
      float x;
      get(k, e, x);
      if (x != -INFINITY) atomicAdd(&h[bin_of(x, M).bin], (unsigned long long)mass_of(x, M));
    }
    __syncthreads();
    if (wave == 0) {
      uint32_t bb;
      uint64_t ab, Z;
      ps_find(h, 0, ~0ull, bb, ab, Z);
      uint32_t b1 = NB1;
      uint64_t T = 0, above1 = 0;
      if (a.top_p[lv] < 1.0f && Z > 0) {
        const double tt = ceil((double)a.top_p[lv] * (double)Z);
        T = tt < 1.0 ? 1ull : (uint64_t)tt;
        if (T > Z) T = Z;
        uint64_t dummy;
        ps_find(h, 0, T, b1, above1, dummy);
      }
      if (lane == 0) { s_b1 = b1; s_T = T; s_above1 = above1; s_ntie = 0; }
    }
    __syncthreads();
    const uint32_t b1 = s_b1;
    const uint64_t T = s_T;
    // ---- nodes of the bins above the boundary bin are kept; the boundary bin's fine histogram
    for (int k = tid; k < NB2; k += PS_THREADS) h[k] = 0ull;
    __syncthreads();
    for (int64_t k = tid; k < count; k += PS_THREADS) {
      int64_t e;
      float x;
      get(k, e, x);
      if (x == -INFINITY) continue;
      const BinSub bs = bin_of(x, M);
      if (bs.bin < b1) atomicOr(&kb[e >> 5], 1u << (e & 31));
      else if (bs.bin == b1) atomicAdd(&h[bs.sub], (unsigned long long)mass_of(x, M));
    }
    __syncthreads();
    if (b1 < (uint32_t)NB1) {
      if (wave == 0) {
        uint32_t b2;
        uint64_t above2, tot;
        ps_find(h, s_above1, T, b2, above2, tot);
        if (lane == 0) { s_b2 = b2; s_above2 = above2; }
      }
      __syncthreads();
      const uint32_t b2 = s_b2;
      const uint64_t above2 = s_above2;
      for (int64_t k = tid; k < count; k += PS_THREADS) {
        int64_t e;
        float x;
        get(k, e, x);
        if (x == -INFINITY) continue;
        const BinSub bs = bin_of(x, M);
        if (bs.bin != b1) continue;
        if (bs.sub < b2) {
          atomicOr(&kb[e >> 5], 1u << (e & 31));
        } else if (bs.sub == b2) {
          const uint32_t j = atomicAdd(&s_ntie, 1u);
          if (j < (uint32_t)PS_TIES) { tie_e[j] = (int32_t)e; tie_s[j] = x; tie_m[j] = mass_of(x, M); }
        }
      }
      __syncthreads();
      const uint32_t nt = s_ntie;
      if (nt <= (uint32_t)PS_TIES) {
        // exact rank order among the boundary sub-bin's nodes: a node is kept while the
        // mass ranked before it is still below the target
        for (uint32_t x = tid; x < nt; x += PS_THREADS) {
          uint64_t ab = 0;
          const uint64_t kx = rank_key(tie_s[x], tie_e[x]);
          for (uint32_t y = 0; y < nt; ++y)
            if (rank_key(tie_s[y], tie_e[y]) < kx) ab += tie_m[y];
          if (above2 + ab < T) atomicOr(&kb[tie_e[x] >> 5], 1u << (tie_e[x] & 31));
        }
      } else {
        // radix select on the 64-bit rank key of the boundary sub-bin's nodes, 8 bits a pass
        unsigned long long* dh = h;
        if (tid == 0) { s_prefix = 0; s_rabove = above2; }
        __syncthreads();
        for (int pass = 0; pass < 8; ++pass) {
          const int shift = 56 - 8 * pass;
          const uint64_t hi = pass == 0 ? 0ull : (~0ull << (shift + 8));
          for (int k = tid; k < 256; k += PS_THREADS) dh[k] = 0ull;
          __syncthreads();
          const uint64_t pf = s_prefix;
          for (int64_t k = tid; k < count; k += PS_THREADS) {
            int64_t e;
            float x;
            get(k, e, x);
            if (x == -INFINITY) continue;
            const BinSub bs = bin_of(x, M);
            if (bs.bin != b1 || bs.sub != b2) continue;
            const uint64_t rk = rank_key(x, (int32_t)e);
            if ((rk & hi) == (pf & hi)) atomicAdd(&dh[(rk >> shift) & 255u], (unsigned long long)mass_of(x, M));
          }
          __syncthreads();
          if (tid == 0) {
            uint64_t run = s_rabove;
            for (int dd = 0; dd < 256; ++dd) {
              if (run + dh[dd] >= T) { s_prefix = pf | ((uint64_t)dd << shift); s_rabove = run; break; }
              run += dh[dd];
            }
          }
          __syncthreads();
        }
        const uint64_t kbnd = s_prefix;
        for (int64_t k = tid; k < count; k += PS_THREADS) {
          int64_t e;
          float x;
          get(k, e, x);
          if (x == -INFINITY) continue;
          const BinSub bs = bin_of(x, M);
          if (bs.bin == b1 && bs.sub == b2 && rank_key(x, (int32_t)e) <= kbnd) atomicOr(&kb[e >> 5], 1u << (e & 31));
        }
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- gather lists
// Per (query, KV head): the level-1 blocks some head of the query kept, with the mask of
// those heads, in block order (256 words of 32 blocks a round, compacted by a block scan).
__global__ __launch_bounds__(256) void prefill_gather_kernel(PrefillArgs a) {
  __shared__ int32_t wsum[4];
  const int i = blockIdx.x, kv = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = a.g;
  const int64_t n = a.nl[1];
  const int64_t nw = (n + 31) >> 5;
  const int64_t cap1 = a.dev.ncap[1];
  int32_t* onode = a.L0node + ((int64_t)i * a.hkv + kv) * cap1;
  uint32_t* omask = a.L0mask + ((int64_t)i * a.hkv + kv) * cap1;
  const uint32_t* kb0 = a.KB + a.koff[1] + ((int64_t)kv * a.P + (int64_t)i * g) * a.kstride[1];
  int32_t base = 0;
  for (int64_t w0 = 0; w0 < nw; w0 += 256) {
    const int64_t w = w0 + tid;
    uint32_t words[GMAX];
    uint32_t any = 0u;
#pragma unroll
    for (int gi = 0; gi < GMAX; ++gi) {
      words[gi] = (gi < g && w < nw) ? kb0[(int64_t)gi * a.kstride[1] + w] : 0u;
      any |= words[gi];
    }
    const int cnt = __popc(any);
    // exclusive scan of the counts over the workgroup
    int inc = cnt;
    for (int off = 1; off < 64; off <<= 1) {
      const int x = __shfl_up(inc, off);
      if (lane >= off) inc += x;
    }
    if (lane == 63) wsum[wave] = inc;
    __syncthreads();
    int off = base + inc - cnt;
    for (int k = 0; k < wave; ++k) off += wsum[k];
    const int32_t round = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    uint32_t rest = any;
    while (rest) {
      const int k = __ffs(rest) - 1;
      rest &= rest - 1u;
      uint32_t mk = 0u;
#pragma unroll
      for (int gi = 0; gi < GMAX; ++gi) mk |= ((words[gi] >> k) & 1u) << gi;
      onode[off] = (int32_t)(32 * w + k);
      omask[off] = mk;
      ++off;
    }
    base += round;
    __syncthreads();
  }
  if (tid == 0) a.cnt0[(int64_t)i * a.hkv + kv] = base;
}

// ---------------------------------------------------------------- launchers
template <typename TIn, int D, int R>
static void launch_prefix_t(const PrefillArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((prefill_prefix_kernel<TIn, D, R>), dim3((unsigned)a.mb, (unsigned)a.hkv), dim3(256), 0, st, a);
}

hipError_t launch_prefill_prefix(const PrefillArgs& a, bool bf16, int D, int R, hipStream_t st) {
#define ZHA_CASE(DD, RR)                                                       \
  if (D == DD && R == RR) {                                                    \
    if (bf16) launch_prefix_t<bf16_t, DD, RR>(a, st);                          \
    else launch_prefix_t<float, DD, RR>(a, st);                                \
    return hipGetLastError();                                                  \
  }
  ZHA_CASE(64, 1) ZHA_CASE(64, 2) ZHA_CASE(64, 4) ZHA_CASE(64, 8) ZHA_CASE(64, 16)
  ZHA_CASE(128, 1) ZHA_CASE(128, 2) ZHA_CASE(128, 4) ZHA_CASE(128, 8) ZHA_CASE(128, 16)
#undef ZHA_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_qprep(const PrefillArgs& a, bool bf16, int D, hipStream_t st) {
  const unsigned grid = grid_for((int64_t)a.mb * a.hq * D, 256, 1024);
  if (bf16) {
    if (D == 64) hipLaunchKernelGGL((prefill_qprep_kernel<bf16_t, 64>), dim3(grid), dim3(256), 0, st, a);
    else hipLaunchKernelGGL((prefill_qprep_kernel<bf16_t, 128>), dim3(grid), dim3(256), 0, st, a);
  } else {
    if (D == 64) hipLaunchKernelGGL((prefill_qprep_kernel<float, 64>), dim3(grid), dim3(256), 0, st, a);
    else hipLaunchKernelGGL((prefill_qprep_kernel<float, 128>), dim3(grid), dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

template <int D, int R>
static void launch_score_t(const PrefillArgs& a, hipStream_t st) {
  static const int per_cu = resident_per_cu(prefill_score_kernel<D, R>, 256);
  const int64_t cap = (int64_t)per_cu * device_cus() / a.hkv;
  hipLaunchKernelGGL((prefill_score_kernel<D, R>), dim3(grid_for(a.nl[1], 4 * (16 / R), cap), (unsigned)a.hkv,
                                                         (unsigned)a.levels), dim3(256), 0, st, a);
}

hipError_t launch_prefill_score(const PrefillArgs& a, int D, int R, hipStream_t st) {
#define ZHA_CASE(DD, RR) if (D == DD && R == RR) { launch_score_t<DD, RR>(a, st); return hipGetLastError(); }
  ZHA_CASE(64, 1) ZHA_CASE(64, 2) ZHA_CASE(64, 4) ZHA_CASE(64, 8) ZHA_CASE(64, 16)
  ZHA_CASE(128, 1) ZHA_CASE(128, 2) ZHA_CASE(128, 4) ZHA_CASE(128, 8) ZHA_CASE(128, 16)
#undef ZHA_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_tail(const PrefillArgs& a, int D, int R, hipStream_t st) {
  const dim3 grid((unsigned)a.P, (unsigned)a.hkv, (unsigned)a.levels);
#define ZHA_CASE(DD, RR)                                                                  \
  if (D == DD && R == RR) {                                                               \
    hipLaunchKernelGGL((prefill_tail_kernel<DD, RR>), grid, dim3(64), 0, st, a);          \
    return hipGetLastError();                                                             \
  }
  ZHA_CASE(64, 1) ZHA_CASE(64, 2) ZHA_CASE(64, 4) ZHA_CASE(64, 8) ZHA_CASE(64, 16)
  ZHA_CASE(128, 1) ZHA_CASE(128, 2) ZHA_CASE(128, 4) ZHA_CASE(128, 8) ZHA_CASE(128, 16)
#undef ZHA_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_select(const PrefillArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(prefill_select_kernel, dim3((unsigned)a.P, (unsigned)a.hkv), dim3(PS_THREADS), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_prefill_gather(const PrefillArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(prefill_gather_kernel, dim3((unsigned)a.mb, (unsigned)a.hkv), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace zha
