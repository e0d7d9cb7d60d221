// Top-down top-p router.
//
// Blog "Zyphra Hierarchical Attention", section "Routing through the tree": a query scores
// the top level, keeps the smallest set of nodes that accounts for a fraction p of the
// estimated attention probability (top-p), expands only those nodes' children and repeats
// down to the raw keys; several branches may stay open.  A node's score is the max over
// its reference planes, max_j(q.s_j/sqrt(d) + c_j) (news summary "Zyphra releases the ZHA
// sparse attention method", section "Building the tree").  Probabilities are the softmax
// of the scores over the current frontier; nodes are ranked by score, equal scores by
// node id; "reaching p" means cumulative probability >= p; p >= 1 keeps everything.
//
// GPU organisation.  The query heads of one GQA group share a KV head, hence a tree; the
// router keeps, per KV head and level, the UNION of the group's frontiers as a node list
// sorted by id with a bitmask of the heads whose frontier holds each node, so a node's
// planes are read once per group.  Per level:
//   score     planes -> scores of all heads of the group; per-head max (ordered-int atomics)
//   hist      per head: fixed-point probability mass (2^40 = probability 1 relative to the
//             head's max) binned by (max - score) in 1/64 steps; integer sums make the
//             result independent of execution order
//   select    per head: scan the bins, find the bin where the cumulative mass reaches
//             ceil(p * Z)
//   classify  nodes above that bin are kept; nodes inside it are collected as candidates
//             and binned again 2048x finer
//   resolve   per head: scan the fine bins; resolve the nodes of the boundary fine bin in
//             exact rank order (pairwise in LDS, or radix select on (score, id) for many)
//   expand    two-pass scan-and-emit of the kept nodes' children (the next union list, in
//             id order), or of the kept level-1 blocks (the gather list)
// Nothing is read back to the host: list sizes live on the device.
#include "common.hpp"
#include "kernels.hpp"

// Score-kernel tuning: tiles in flight per wave (R >= 8 / R < 8) and max blocks per KV head.
#ifndef ZHA_SCORE_UN_WIDE
#define ZHA_SCORE_UN_WIDE 2
#endif
#ifndef ZHA_SCORE_UN_NARROW
#define ZHA_SCORE_UN_NARROW 2
#endif
#ifndef ZHA_SCORE_GRID
#define ZHA_SCORE_GRID 1024
#endif

namespace zha {

template <typename TIn, int D>
__global__ __launch_bounds__(256) void route_prep_kernel(RouteArgs a) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t nth = (int64_t)gridDim.x * blockDim.x;
  const TIn* q = (const TIn*)a.q;
  for (int64_t i = tid; i < (int64_t)a.hq * D; i += nth) a.dev.qf[i] = a.sigma * to_f32(q[i]);
  const int64_t nq = (int64_t)(a.levels + 1) * a.hq;
  for (int64_t i = tid; i < nq; i += nth) {
    QState z = {};
    a.dev.qs[i] = z;
  }
  for (int64_t i = tid; i < nq * NB1; i += nth) a.dev.mass1[i] = 0;
  for (int64_t i = tid; i < nq * NB2; i += nth) a.dev.mass2[i] = 0;
  const int L = a.levels;
  const int64_t capL = a.dev.ncap[L];
  const uint32_t full = (a.g >= 32) ? 0xffffffffu : ((1u << a.g) - 1u);
  for (int64_t i = tid; i < (int64_t)a.hkv * a.nlevel; i += nth) {
    const int64_t kv = i / a.nlevel, n = i % a.nlevel;
    a.dev.node[L][kv * capL + n] = (int32_t)n;
    a.dev.mask[L][kv * capL + n] = full;
  }
  for (int64_t i = tid; i < (int64_t)(MAXL + 1) * a.hkv; i += nth)
    a.dev.cnt[i] = (i / a.hkv == L) ? (int32_t)a.nlevel : 0;
}

// ------------------------------------------------------------------ score
// Scores of the union frontier on fp32 MFMA: one 16x16 output tile = the 16 query-head rows
// (the group's heads, zero-padded) x 16 columns = 16/R nodes x R planes.  The contraction
// over d is permuted so that lane (column c, group kg) streams the contiguous 64-byte
// pieces [64i + 16kg, +16) of its plane row; Q uses the same permutation.  A node's score is
// the max over its R columns (plus the offsets c_j), taken across the R lanes of the node.
template <int D, int R>
__global__ __launch_bounds__(256) void route_score_kernel(RouteArgs a) {
  constexpr int NPT = 16 / R;                 // nodes per 16-column tile
  constexpr int NI = D / 16;                  // float4 loads per lane per tile
  constexpr int UN = R >= 8 ? ZHA_SCORE_UN_WIDE : ZHA_SCORE_UN_NARROW;   // tiles in flight per wave
  __shared__ float red[4][16];
  const int kv = blockIdx.y, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, kg = lane >> 4;
  const int slot = col / R, plane = col % R;
  const int lv = a.level;
  const int64_t cnt = a.dev.cnt[lv * a.hkv + kv];
  const int64_t cap = a.dev.ncap[lv];
  const int32_t* nodes = a.dev.node[lv] + kv * cap;
  const uint32_t* masks = a.dev.mask[lv] + kv * cap;
  const float* S = a.dev.s[lv] + (int64_t)kv * cap * R * D;
  const float* C = a.dev.c[lv] + (int64_t)kv * cap * R;
  float* out = a.dev.score[lv] + (int64_t)kv * GMAX * cap;
  const int g = a.g;

  float qa[NI][4];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
    if (col < g) x = *(const float4*)(a.dev.qf + (int64_t)(kv * g + col) * D + 16 * i + 4 * kg);
    qa[i][0] = x.x; qa[i][1] = x.y; qa[i][2] = x.z; qa[i][3] = x.w;
  }
  float runmax[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};

  const int64_t ntiles = (cnt + NPT - 1) / NPT;
  for (int64_t t0 = ((int64_t)blockIdx.x * 4 + wave) * UN; t0 < ntiles; t0 += (int64_t)gridDim.x * 4 * UN) {
    float4 sb[UN][NI];
    float cj[UN];
    int64_t ent[UN];
    bool ok[UN];
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      ent[u] = (t0 + u) * NPT + slot;
      ok[u] = (t0 + u) < ntiles && ent[u] < cnt;
      const int64_t nid = ok[u] ? nodes[ent[u]] : 0;
      const float* sp = S + (nid * R + plane) * D + 4 * kg;
#pragma unroll
      for (int i = 0; i < NI; ++i) sb[u][i] = ok[u] ? *(const float4*)(sp + 16 * i) : make_float4(0.f, 0.f, 0.f, 0.f);
      cj[u] = ok[u] ? C[nid * R + plane] : -INFINITY;
    }
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[i][0], sb[u][i].x, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[i][1], sb[u][i].y, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[i][2], sb[u][i].z, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[i][3], sb[u][i].w, acc, 0, 0, 0);
      }
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = acc[e] + cj[u];
#pragma unroll
      for (int off = 1; off < R; off <<= 1)
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = fmaxf(v[e], __shfl_xor(v[e], off));
      const uint32_t mk = ok[u] ? masks[ent[u]] : 0u;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int h = kg * 4 + e;
        if (ok[u] && plane == 0 && h < g) out[(int64_t)h * cap + ent[u]] = v[e];
        if ((mk >> h) & 1u) runmax[e] = fmaxf(runmax[e], v[e]);
      }
    }
  }
  // per-head max: lanes of one 16-lane row share kg, i.e. the heads 4kg..4kg+3
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float v = runmax[e];
    for (int off = 1; off < 16; off <<= 1) v = fmaxf(v, __shfl_xor(v, off));
    if (col == 0) red[wave][kg * 4 + e] = v;
  }
  __syncthreads();
  if (threadIdx.x < g) {
    const int gi = threadIdx.x;
    const float m = fmaxf(fmaxf(red[0][gi], red[1][gi]), fmaxf(red[2][gi], red[3][gi]));
    if (m > -INFINITY) atomicMax(&a.dev.qs[lv * a.hq + kv * g + gi].maxkey, f2key(m));
  }
}

// ------------------------------------------------------------------ histogram
__global__ __launch_bounds__(256) void route_hist_kernel(RouteArgs a) {
  __shared__ unsigned long long h[NB1];
  const int hq = blockIdx.y, kv = hq / a.g, gi = hq % a.g, lv = a.level;
  const uint32_t mk = a.dev.qs[lv * a.hq + hq].maxkey;
  if (mk == 0u) return;   // empty frontier for this head
  for (int i = threadIdx.x; i < NB1; i += 256) h[i] = 0ull;
  __syncthreads();
  const float M = key2f(mk);
  const int64_t cnt = a.dev.cnt[lv * a.hkv + kv];
  const int64_t cap = a.dev.ncap[lv];
  const uint32_t* masks = a.dev.mask[lv] + kv * cap;
  const float* sc = a.dev.score[lv] + ((int64_t)kv * GMAX + gi) * cap;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < cnt; e += (int64_t)gridDim.x * 256) {
    if ((masks[e] >> gi) & 1u) {
      BinMass bm = bin_mass(sc[e], M);
      atomicAdd(&h[bm.bin], (unsigned long long)bm.mass);
    }
  }
  __syncthreads();
  unsigned long long* gh = (unsigned long long*)a.dev.mass1 + (int64_t)(lv * a.hq + hq) * NB1;
  for (int i = threadIdx.x; i < NB1; i += 256)
    if (h[i]) atomicAdd(&gh[i], h[i]);
}

// Block-wide scan of NB (=2048) u64 bins held 8 per thread; finds the first bin where
// base + inclusive prefix >= target.  Returns (bin, mass before it) via LDS.
__device__ void find_boundary(const uint64_t* bins, uint64_t base, uint64_t target, uint64_t* tsum,
                              uint32_t* out_bin, uint64_t* out_above, uint64_t* out_total) {
  const int t = threadIdx.x;
  uint64_t v[8];
  uint64_t s = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) { v[i] = bins[t * 8 + i]; s += v[i]; }
  tsum[t] = s;
  __syncthreads();
  // inclusive scan over 256 thread sums (Hillis-Steele in LDS)
  for (int off = 1; off < 256; off <<= 1) {
    uint64_t add = t >= off ? tsum[t - off] : 0ull;
    __syncthreads();
    tsum[t] += add;
    __syncthreads();
  }
  uint64_t run = base + (t ? tsum[t - 1] : 0ull);
  if (t == 255 && out_total) *out_total = tsum[255];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (run < target && run + v[i] >= target) {
      *out_bin = (uint32_t)(t * 8 + i);
      *out_above = run;
    }
    run += v[i];
  }
  __syncthreads();
}

__global__ __launch_bounds__(256) void route_select_kernel(RouteArgs a) {
  __shared__ uint64_t tsum[256];
  __shared__ uint32_t bin;
  __shared__ uint64_t above, total;
  const int hq = blockIdx.x, lv = a.level;
  QState* qs = a.dev.qs + lv * a.hq + hq;
  const uint64_t* bins = a.dev.mass1 + (int64_t)(lv * a.hq + hq) * NB1;
  if (threadIdx.x == 0) { bin = NB1; above = 0; total = 0; }
  __syncthreads();
  // total first (target depends on it)
  find_boundary(bins, 0, ~0ull, tsum, &bin, &above, &total);
  const uint64_t Z = total;
  uint64_t T = 0;
  bool keep_all = a.top_p >= 1.0f || qs->maxkey == 0u || Z == 0;
  if (!keep_all) {
    double t = ceil((double)a.top_p * (double)Z);
    T = t < 1.0 ? 1ull : (uint64_t)t;
    if (T > Z) T = Z;
    if (threadIdx.x == 0) { bin = NB1; above = 0; }
    __syncthreads();
    find_boundary(bins, 0, T, tsum, &bin, &above, nullptr);
  }
  if (threadIdx.x == 0) {
    qs->total = Z;
    qs->target = T;
    qs->b1 = keep_all ? (uint32_t)NB1 : bin;
    qs->above1 = keep_all ? 0ull : above;
  }
}

// ------------------------------------------------------------------ classify
__global__ __launch_bounds__(256) void route_classify_kernel(RouteArgs a) {
  __shared__ float Ms[GMAX];
  __shared__ uint32_t B1[GMAX];
  const int kv = blockIdx.y, lv = a.level, g = a.g;
  if (threadIdx.x < GMAX) {
    const int gi = threadIdx.x;
    if (gi < g) {
      const QState* qs = a.dev.qs + lv * a.hq + kv * g + gi;
      Ms[gi] = key2f(qs->maxkey);
      B1[gi] = qs->b1;
    }
  }
  __syncthreads();
  const int64_t cnt = a.dev.cnt[lv * a.hkv + kv];
  const int64_t cap = a.dev.ncap[lv];
  const uint32_t* masks = a.dev.mask[lv] + kv * cap;
  const float* sc = a.dev.score[lv] + (int64_t)kv * GMAX * cap;
  uint32_t* keep = a.dev.keep[lv] + kv * cap;
  const int64_t ccap = a.dev.ncap[1];
  const int lane = threadIdx.x & 63;
  // wave-uniform trip count so every lane takes part in the candidate ballots
  for (int64_t eb = (int64_t)blockIdx.x * 256 + (threadIdx.x & ~63); eb < cnt; eb += (int64_t)gridDim.x * 256) {
    const int64_t e = eb + lane;
    const bool valid = e < cnt;
    const uint32_t mk = valid ? masks[e] : 0u;
    uint32_t kb = 0;
    for (int gi = 0; gi < g; ++gi) {
      bool cand = false;
      uint64_t cmass = 0;
      uint32_t csub = 0;
      if ((mk >> gi) & 1u) {
        if (B1[gi] >= (uint32_t)NB1) {
          kb |= 1u << gi;
        } else {
          BinMass bm = bin_mass(sc[(int64_t)gi * cap + e], Ms[gi]);
          if (bm.bin < B1[gi]) kb |= 1u << gi;
          else if (bm.bin == B1[gi]) { cand = true; cmass = bm.mass; csub = bm.sub; }
        }
      }
      const uint64_t ball = __ballot(cand);
      if (ball) {
        const int hq = kv * g + gi;
        uint32_t base = 0;
        if (lane == 0) base = atomicAdd(&a.dev.qs[lv * a.hq + hq].ncand, (uint32_t)__popcll(ball));
        base = __shfl(base, 0);
        if (cand) {
          const uint32_t pos = base + (uint32_t)__popcll(ball & ((1ull << lane) - 1ull));
          a.dev.cand[(int64_t)hq * ccap + pos] = (int32_t)e;
          atomicAdd((unsigned long long*)a.dev.mass2 + (int64_t)(lv * a.hq + hq) * NB2 + csub,
                    (unsigned long long)cmass);
        }
      }
    }
    if (valid) keep[e] = kb;
  }
}

// ------------------------------------------------------------------ resolve
__device__ __forceinline__ void wave_sync_lds_r() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint64_t rank_key(float s, int32_t e) {
  return ((uint64_t)(~f2key(s)) << 32) | (uint32_t)e;   // ascending = rank order
}

__global__ __launch_bounds__(256) void route_resolve_kernel(RouteArgs a) {
  __shared__ uint64_t tsum[256];
  __shared__ uint32_t bin;
  __shared__ uint64_t above;
  __shared__ int32_t tie_e[CAND_PAIRWISE];
  __shared__ float tie_s[CAND_PAIRWISE];
  __shared__ uint64_t tie_m[CAND_PAIRWISE];
  __shared__ uint32_t ntie;
  __shared__ unsigned long long dh[256];
  __shared__ uint64_t prefix, rabove;
  const int hq = blockIdx.x, lv = a.level, kv = hq / a.g, gi = hq % a.g;
  QState* qs = a.dev.qs + lv * a.hq + hq;
  const uint32_t b1 = qs->b1;
  if (b1 >= (uint32_t)NB1) return;
  const uint64_t T = qs->target, above1 = qs->above1;
  const float M = key2f(qs->maxkey);
  if (threadIdx.x == 0) { bin = NB2; above = 0; ntie = 0; }
  __syncthreads();
  find_boundary(a.dev.mass2 + (int64_t)(lv * a.hq + hq) * NB2, above1, T, tsum, &bin, &above, nullptr);
  const uint32_t b2 = bin;
  const uint64_t above2 = above;
  const int64_t cap = a.dev.ncap[lv];
  const float* sc = a.dev.score[lv] + ((int64_t)kv * GMAX + gi) * cap;
  uint32_t* keep = a.dev.keep[lv] + kv * cap;
  const int32_t* cand = a.dev.cand + (int64_t)hq * a.dev.ncap[1];
  const uint32_t ncand = qs->ncand;
  const uint32_t bit = 1u << gi;
  for (uint32_t i = threadIdx.x; i < ncand; i += 256) {
    const int32_t e = cand[i];
    const float s = sc[e];
    BinMass bm = bin_mass(s, M);
    if (bm.sub < b2) {
      atomicOr(&keep[e], bit);
    } else if (bm.sub == b2) {
      const uint32_t k = atomicAdd(&ntie, 1u);
      if (k < (uint32_t)CAND_PAIRWISE) { tie_e[k] = e; tie_s[k] = s; tie_m[k] = bm.mass; }
    }
  }
  __syncthreads();
  const uint32_t nt = ntie;
  if (nt <= (uint32_t)CAND_PAIRWISE) {
    for (uint32_t x = threadIdx.x; x < nt; x += 256) {
      uint64_t ab = 0;
      const uint64_t kx = rank_key(tie_s[x], tie_e[x]);
      for (uint32_t y = 0; y < nt; ++y)
        if (rank_key(tie_s[y], tie_e[y]) < kx) ab += tie_m[y];
      if (above2 + ab < T) atomicOr(&keep[tie_e[x]], bit);
    }
  } else {
    // Radix select on the 64-bit rank key of the boundary sub-bin's nodes, 8 bits a pass.
    if (threadIdx.x == 0) { prefix = 0; rabove = above2; }
    __syncthreads();
    for (int pass = 0; pass < 8; ++pass) {
      const int shift = 56 - 8 * pass;
      const uint64_t hi = pass == 0 ? 0ull : (~0ull << (shift + 8));
      dh[threadIdx.x] = 0ull;
      __syncthreads();
      const uint64_t pf = prefix;
      for (uint32_t i = threadIdx.x; i < ncand; i += 256) {
        const int32_t e = cand[i];
        const float s = sc[e];
        BinMass bm = bin_mass(s, M);
        if (bm.sub != b2) continue;
        const uint64_t k = rank_key(s, e);
        if ((k & hi) == (pf & hi)) atomicAdd(&dh[(k >> shift) & 255u], (unsigned long long)bm.mass);
      }
      __syncthreads();
      if (threadIdx.x == 0) {
        uint64_t run = rabove;
        for (int d = 0; d < 256; ++d) {
          if (run + dh[d] >= T) { prefix = pf | ((uint64_t)d << shift); rabove = run; break; }
          run += dh[d];
        }
      }
      __syncthreads();
    }
    const uint64_t kb = prefix;
    for (uint32_t i = threadIdx.x; i < ncand; i += 256) {
      const int32_t e = cand[i];
      const float s = sc[e];
      BinMass bm = bin_mass(s, M);
      if (bm.sub == b2 && rank_key(s, e) <= kb) atomicOr(&keep[e], bit);
    }
  }
  if (threadIdx.x == 0) {
    qs->b2 = b2;
    qs->above2 = above2;
    qs->nties = nt;
    qs->flags = nt > (uint32_t)CAND_PAIRWISE ? 1u : 0u;
  }
}

// ------------------------------------------------------------------ expand
__device__ __forceinline__ int emitted(const RouteArgs& a, int64_t node, uint32_t kb) {
  if (!kb) return 0;
  if (a.level == 1) return 1;
  const int64_t first = node * a.b;
  const int64_t n = a.nbelow - first;
  return (int)(n < a.b ? n : a.b);
}

__global__ __launch_bounds__(256) void route_expand_count_kernel(RouteArgs a) {
  __shared__ int32_t red[4];
  const int kv = blockIdx.y, lv = a.level;
  const int64_t cnt = a.dev.cnt[lv * a.hkv + kv];
  const int64_t cap = a.dev.ncap[lv];
  const int64_t e0 = (int64_t)blockIdx.x * EXPAND_CHUNK;
  int32_t c = 0;
  for (int64_t e = e0 + threadIdx.x; e < min(cnt, e0 + EXPAND_CHUNK); e += 256)
    c += emitted(a, a.dev.node[lv][kv * cap + e], a.dev.keep[lv][kv * cap + e]);
  for (int off = 1; off < 64; off <<= 1) c += __shfl_xor(c, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0)
    a.dev.part[lv][(int64_t)kv * gridDim.x + blockIdx.x] = red[0] + red[1] + red[2] + red[3];
}

__global__ __launch_bounds__(256) void route_expand_emit_kernel(RouteArgs a) {
  __shared__ int32_t red[4], red2[4];
  __shared__ int32_t ts[256];
  __shared__ int32_t eoff[EXPAND_CHUNK + 1];   // exclusive output offset of each entry
  __shared__ int32_t enode[EXPAND_CHUNK];
  __shared__ uint32_t ekeep[EXPAND_CHUNK];
  const int kv = blockIdx.y, lv = a.level;
  const int64_t cnt = a.dev.cnt[lv * a.hkv + kv];
  const int64_t cap = a.dev.ncap[lv];
  const int nch = gridDim.x;
  const int32_t* part = a.dev.part[lv] + (int64_t)kv * nch;
  // offset of this chunk (and the grand total, written by chunk 0)
  int32_t pre = 0, tot = 0;
  for (int i = threadIdx.x; i < nch; i += 256) {
    const int32_t v = part[i];
    tot += v;
    if (i < (int)blockIdx.x) pre += v;
  }
  for (int off = 1; off < 64; off <<= 1) {
    pre += __shfl_xor(pre, off);
    tot += __shfl_xor(tot, off);
  }
  if ((threadIdx.x & 63) == 0) { red[threadIdx.x >> 6] = pre; red2[threadIdx.x >> 6] = tot; }
  // each thread owns 4 consecutive entries of the chunk
  const int64_t c0 = (int64_t)blockIdx.x * EXPAND_CHUNK;
  int32_t cnt4[4];
  int32_t mine = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int j = threadIdx.x * 4 + i;
    const int64_t e = c0 + j;
    int32_t nd = 0;
    uint32_t kb = 0;
    cnt4[i] = 0;
    if (e < cnt) {
      nd = a.dev.node[lv][kv * cap + e];
      kb = a.dev.keep[lv][kv * cap + e];
      cnt4[i] = emitted(a, nd, kb);
    }
    enode[j] = nd;
    ekeep[j] = kb;
    mine += cnt4[i];
  }
  ts[threadIdx.x] = mine;
  __syncthreads();
  const int32_t base = red[0] + red[1] + red[2] + red[3];
  const int out_lv = lv - 1;
  if (blockIdx.x == 0 && threadIdx.x == 0)
    a.dev.cnt[out_lv * a.hkv + kv] = red2[0] + red2[1] + red2[2] + red2[3];
  for (int off = 1; off < 256; off <<= 1) {
    const int32_t add = threadIdx.x >= off ? ts[threadIdx.x - off] : 0;
    __syncthreads();
    ts[threadIdx.x] += add;
    __syncthreads();
  }
  int32_t run = ts[threadIdx.x] - mine;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    eoff[threadIdx.x * 4 + i] = run;
    run += cnt4[i];
  }
  if (threadIdx.x == 255) eoff[EXPAND_CHUNK] = ts[255];
  __syncthreads();
  // coalesced emission: consecutive threads write consecutive output slots
  const int32_t total = eoff[EXPAND_CHUNK];
  const int64_t ocap = a.dev.ncap[out_lv];
  int32_t* onode = a.dev.node[out_lv] + kv * ocap + base;
  uint32_t* omask = a.dev.mask[out_lv] + kv * ocap + base;
  for (int32_t o = threadIdx.x; o < total; o += 256) {
    int lo = 0, hi = EXPAND_CHUNK - 1;   // last entry j with eoff[j] <= o
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (eoff[mid] <= o) lo = mid; else hi = mid - 1;
    }
    const int32_t c = o - eoff[lo];
    onode[o] = lv == 1 ? enode[lo] : enode[lo] * a.b + c;
    omask[o] = ekeep[lo];
  }
}

// ------------------------------------------------------------------ launchers
hipError_t launch_route_prep(const RouteArgs& a, bool bf16, int D, hipStream_t st) {
  dim3 grid(256), block(256);
  if (bf16) {
    if (D == 64) hipLaunchKernelGGL((route_prep_kernel<bf16_t, 64>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((route_prep_kernel<bf16_t, 128>), grid, block, 0, st, a);
  } else {
    if (D == 64) hipLaunchKernelGGL((route_prep_kernel<float, 64>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((route_prep_kernel<float, 128>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

template <int D, int R>
static void launch_score(const RouteArgs& a, hipStream_t st) {
  constexpr int NPB = 4 * (16 / R) * (R >= 8 ? ZHA_SCORE_UN_WIDE : ZHA_SCORE_UN_NARROW);   // nodes per block pass
  int64_t x = (a.nlevel + NPB - 1) / NPB;
  if (x > ZHA_SCORE_GRID) x = ZHA_SCORE_GRID;
  if (x < 1) x = 1;
  hipLaunchKernelGGL((route_score_kernel<D, R>), dim3((unsigned)x, (unsigned)a.hkv), dim3(256), 0, st, a);
}

static unsigned grid_for(int64_t n, int64_t per, int64_t cap) {
  int64_t x = (n + per - 1) / per;
  if (x > cap) x = cap;
  return (unsigned)(x < 1 ? 1 : x);
}

hipError_t launch_route_score(const RouteArgs& a, int D, int R, hipStream_t st) {
#define ZHA_CASE(DD, RR) else if (D == DD && R == RR) launch_score<DD, RR>(a, st);
  if (false) {}
  ZHA_CASE(64, 1) ZHA_CASE(64, 2) ZHA_CASE(64, 4) ZHA_CASE(64, 8) ZHA_CASE(64, 16)
  ZHA_CASE(128, 1) ZHA_CASE(128, 2) ZHA_CASE(128, 4) ZHA_CASE(128, 8) ZHA_CASE(128, 16)
  else return hipErrorInvalidValue;
#undef ZHA_CASE
  return hipGetLastError();
}

hipError_t launch_route_select(const RouteArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(route_hist_kernel, dim3(grid_for(a.nlevel, 2048, 256), (unsigned)a.hq), dim3(256), 0, st, a);
  hipLaunchKernelGGL(route_select_kernel, dim3((unsigned)a.hq), dim3(256), 0, st, a);
  hipLaunchKernelGGL(route_classify_kernel, dim3(grid_for(a.nlevel, 1024, 2048), (unsigned)a.hkv), dim3(256), 0, st, a);
  hipLaunchKernelGGL(route_resolve_kernel, dim3((unsigned)a.hq), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_route_expand(const RouteArgs& a, hipStream_t st) {
  const unsigned nch = (unsigned)((a.nlevel + EXPAND_CHUNK - 1) / EXPAND_CHUNK);
  dim3 grid(nch < 1 ? 1 : nch, (unsigned)a.hkv);
  hipLaunchKernelGGL(route_expand_count_kernel, grid, dim3(256), 0, st, a);
  hipLaunchKernelGGL(route_expand_emit_kernel, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace zha
