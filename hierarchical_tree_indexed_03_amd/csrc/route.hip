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
  const bool dense = a.dense != 0;            // every node of the level, no list
  const int lv = dense ? a.level - (int)blockIdx.z : a.level;
  const int64_t cnt = dense ? a.nl[lv] : a.dev.cnt[lv * a.hkv + kv];
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
      const int64_t nid = ok[u] ? (dense ? ent[u] : (int64_t)nodes[ent[u]]) : 0;
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
      const uint32_t mk = (ok[u] && !dense) ? masks[ent[u]] : 0u;   // dense: max taken later
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
// Large levels pick each head's top-p set in four launches: partial coarse histograms
// (hist), their reduction and the boundary bin (bound), keep / candidate classification
// (classify) and the exact decision inside the boundary bin (resolve).  No step needs a
// contended global atomic: partial histograms are plain stores and candidates are appended
// in per-workgroup batches.
constexpr int SEL_THREADS = 512;
constexpr int HIST_U = 2;          // union entries per thread per iteration (loads issued together)
constexpr int CAND_STAGE = 1024;   // candidates staged per head in LDS before a batch append

// Each workgroup takes a contiguous range of the KV head's union list, reads every entry's
// mask once and adds the node's mass to the coarse histogram of every head of the group
// that has it in its frontier; the workgroup's histograms are stored whole.
__global__ __launch_bounds__(SEL_THREADS) void route_hist_kernel(RouteArgs a) {
  __shared__ unsigned long long h[GMAX][NB1];
  __shared__ float Ms[GMAX];
  const int kv = blockIdx.y, lv = a.level, g = a.g;
  if (threadIdx.x < GMAX) {
    const uint32_t mk = threadIdx.x < g ? a.dev.qs[lv * a.hq + kv * g + threadIdx.x].maxkey : 0u;
    Ms[threadIdx.x] = mk ? key2f(mk) : -INFINITY;
  }
  for (int i = threadIdx.x; i < GMAX * NB1; i += SEL_THREADS) (&h[0][0])[i] = 0ull;
  __syncthreads();
  const int64_t cnt = a.dev.cnt[lv * a.hkv + kv];
  const int64_t cap = a.dev.ncap[lv];
  const int64_t per = (cnt + gridDim.x - 1) / gridDim.x;
  const int64_t lo = (int64_t)blockIdx.x * per, hi = lo + per < cnt ? lo + per : cnt;
  const uint32_t* masks = a.dev.mask[lv] + kv * cap;
  const float* sc = a.dev.score[lv] + (int64_t)kv * GMAX * cap;
  for (int64_t e0 = lo + threadIdx.x; e0 < hi; e0 += SEL_THREADS * HIST_U) {
    uint32_t mk[HIST_U];
    float v[HIST_U][GMAX];
#pragma unroll
    for (int u = 0; u < HIST_U; ++u) {
      const int64_t e = e0 + SEL_THREADS * u;
      mk[u] = e < hi ? masks[e] : 0u;
      // score rows exist for all GMAX heads; only entries with the head's bit are used
#pragma unroll
      for (int gi = 0; gi < GMAX; ++gi) v[u][gi] = (gi < g && e < hi) ? sc[(int64_t)gi * cap + e] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < HIST_U; ++u)
#pragma unroll
      for (int gi = 0; gi < GMAX; ++gi)
        if ((mk[u] >> gi) & 1u) {
          const BinMass bm = bin_mass(v[u][gi], Ms[gi]);
          atomicAdd(&h[gi][bm.bin], (unsigned long long)bm.mass);
        }
  }
  __syncthreads();
  uint64_t* out = a.dev.hpart + ((int64_t)kv * SEL_P + blockIdx.x) * GMAX * NB1;
  for (int i = threadIdx.x; i < g * NB1; i += SEL_THREADS) out[i] = (&h[0][0])[i];
}

// First bin (of 512 held 8 per lane) where base + inclusive prefix >= target; one wave.
__device__ void wave_boundary512(const uint64_t* bins, uint64_t base, uint64_t target, int lane, uint32_t& bin,
                                 uint64_t& above, uint64_t& total) {
  uint64_t v[8], loc = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) { v[i] = bins[lane * 8 + i]; loc += v[i]; }
  uint64_t inc = loc;
  for (int off = 1; off < 64; off <<= 1) {
    const uint64_t t = __shfl_up(inc, off);
    if (lane >= off) inc += t;
  }
  total = __shfl(inc, 63);
  uint64_t run = base + inc - loc;
  uint32_t fb = 0xffffffffu;
  uint64_t fa = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (fb == 0xffffffffu && run < target && run + v[i] >= target) { fb = lane * 8 + i; fa = run; }
    run += v[i];
  }
  const uint64_t hit = __ballot(fb != 0xffffffffu);
  const int src = hit ? __ffsll((long long)hit) - 1 : 0;
  bin = __shfl(fb, src);
  above = __shfl(fa, src);
}

// One workgroup per query head: sums the partial histograms bin by bin (fixed order) and
// finds the boundary bin of the target mass ceil(p * Z).
__global__ __launch_bounds__(NB1) void route_bound_kernel(RouteArgs a) {
  __shared__ uint64_t hs[NB1];
  const int hq = blockIdx.x, lv = a.level, kv = hq / a.g, gi = hq % a.g;
  QState* qs = a.dev.qs + lv * a.hq + hq;
  if (qs->maxkey == 0u) return;
  const uint64_t* src = a.dev.hpart + ((int64_t)kv * SEL_P * GMAX + gi) * NB1 + threadIdx.x;
  uint64_t sum = 0;
  int p = 0;
  for (; p + 8 <= a.sel_p; p += 8) {
    uint64_t v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = src[(int64_t)(p + i) * GMAX * NB1];
#pragma unroll
    for (int i = 0; i < 8; ++i) sum += v[i];
  }
  for (; p < a.sel_p; ++p) sum += src[(int64_t)p * GMAX * NB1];
  hs[threadIdx.x] = sum;
  __syncthreads();
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  uint32_t bb;
  uint64_t above1, Z, dummy;
  wave_boundary512(hs, 0, ~0ull, lane, bb, above1, Z);
  uint32_t b1 = NB1;
  uint64_t T = 0;
  above1 = 0;
  if (a.top_p < 1.0f && Z > 0) {
    const double tt = ceil((double)a.top_p * (double)Z);
    T = tt < 1.0 ? 1ull : (uint64_t)tt;
    if (T > Z) T = Z;
    wave_boundary512(hs, 0, T, lane, bb, above1, dummy);
    b1 = bb;
  }
  if (lane == 0) {
    qs->total = Z;
    qs->target = T;
    qs->b1 = b1;
    qs->above1 = above1;
  }
}

// ------------------------------------------------------------------ classify
__device__ __forceinline__ void wave_sync_lds_c() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

constexpr int CLS_U = 2;          // union entries per lane per iteration
constexpr int WAVE_STAGE = 128;   // candidates staged per (wave, head) in LDS

// Nodes above the boundary bin are kept; nodes inside it become candidates.  Each wave
// stages its candidates per head in LDS (spilling a batch to the head's list only when its
// stage passes half full); at the end the workgroup appends what its waves hold with one
// atomic per head.
__global__ __launch_bounds__(SEL_THREADS) void route_classify_kernel(RouteArgs a) {
  constexpr int NW = SEL_THREADS / 64;
  __shared__ float Ms[GMAX];
  __shared__ uint32_t B1[GMAX];
  __shared__ int32_t stage[NW][GMAX][WAVE_STAGE];
  __shared__ uint32_t wcnt_s[NW][GMAX];
  __shared__ uint32_t bbase[GMAX];
  const int kv = blockIdx.y, lv = a.level, g = a.g;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (threadIdx.x < GMAX) {
    uint32_t mk = 0, b1 = NB1;
    if (threadIdx.x < g) {
      const QState* qs = a.dev.qs + lv * a.hq + kv * g + threadIdx.x;
      mk = qs->maxkey;
      b1 = mk ? qs->b1 : NB1;
    }
    Ms[threadIdx.x] = mk ? key2f(mk) : -INFINITY;
    B1[threadIdx.x] = b1;
  }
  __syncthreads();
  const int64_t cnt = a.dev.cnt[lv * a.hkv + kv];
  const int64_t cap = a.dev.ncap[lv];
  const int64_t per = (cnt + gridDim.x - 1) / gridDim.x;
  const int64_t lo = (int64_t)blockIdx.x * per, hi = lo + per < cnt ? lo + per : cnt;
  const uint32_t* masks = a.dev.mask[lv] + kv * cap;
  const float* sc = a.dev.score[lv] + (int64_t)kv * GMAX * cap;
  uint32_t* keep = a.dev.keep[lv] + kv * cap;
  const int64_t ccap = a.dev.ncap[1];
  uint32_t wcnt[GMAX];
#pragma unroll
  for (int gi = 0; gi < GMAX; ++gi) wcnt[gi] = 0;
  // wave-uniform trip count so every lane takes part in the ballots
  for (int64_t e0 = lo + (int64_t)wave * 64 * CLS_U; e0 < hi; e0 += SEL_THREADS * CLS_U) {
    uint32_t mk[CLS_U];
    float v[CLS_U][GMAX];
#pragma unroll
    for (int u = 0; u < CLS_U; ++u) {
      const int64_t e = e0 + 64 * u + lane;
      mk[u] = e < hi ? masks[e] : 0u;
#pragma unroll
      for (int gi = 0; gi < GMAX; ++gi) v[u][gi] = (gi < g && e < hi) ? sc[(int64_t)gi * cap + e] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < CLS_U; ++u) {
      const int64_t e = e0 + 64 * u + lane;
      uint32_t kb = 0;
#pragma unroll
      for (int gi = 0; gi < GMAX; ++gi) {
        bool cand = false;
        if ((mk[u] >> gi) & 1u) {
          if (B1[gi] >= (uint32_t)NB1) {
            kb |= 1u << gi;
          } else {
            const BinMass bm = bin_mass(v[u][gi], Ms[gi]);
            if (bm.bin < B1[gi]) kb |= 1u << gi;
            else cand = bm.bin == B1[gi];
          }
        }
        const uint64_t ball = __ballot(cand);
        if (ball) {
          if (cand) stage[wave][gi][wcnt[gi] + __popcll(ball & ((1ull << lane) - 1ull))] = (int32_t)e;
          wcnt[gi] += (uint32_t)__popcll(ball);
          if (wcnt[gi] > WAVE_STAGE - 64) {   // spill this wave's batch for the head
            wave_sync_lds_c();
            uint32_t base = 0;
            if (lane == 0) base = atomicAdd(&a.dev.qs[lv * a.hq + kv * g + gi].ncand, wcnt[gi]);
            base = __shfl(base, 0);
            int32_t* dst = a.dev.cand + (int64_t)(kv * g + gi) * ccap + base;
            for (uint32_t i = lane; i < wcnt[gi]; i += 64) dst[i] = stage[wave][gi][i];
            wave_sync_lds_c();
            wcnt[gi] = 0;
          }
        }
      }
      if (e < hi) keep[e] = kb;
    }
  }
  if (lane < GMAX) wcnt_s[wave][lane] = 0;
#pragma unroll
  for (int gi = 0; gi < GMAX; ++gi)
    if (lane == gi) wcnt_s[wave][gi] = wcnt[gi];
  __syncthreads();
  if (threadIdx.x < (unsigned)g) {
    uint32_t n = 0;
    for (int w = 0; w < NW; ++w) n += wcnt_s[w][threadIdx.x];
    bbase[threadIdx.x] = n ? atomicAdd(&a.dev.qs[lv * a.hq + kv * g + threadIdx.x].ncand, n) : 0u;
  }
  __syncthreads();
  for (int gi = 0; gi < g; ++gi) {
    uint32_t off = bbase[gi];
    for (int w = 0; w < wave; ++w) off += wcnt_s[w][gi];
    int32_t* dst = a.dev.cand + (int64_t)(kv * g + gi) * ccap + off;
    for (uint32_t i = lane; i < wcnt_s[wave][gi]; i += 64) dst[i] = stage[wave][gi][i];
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
  __shared__ unsigned long long h2[NB2];
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
  if (qs->maxkey == 0u || b1 >= (uint32_t)NB1) return;
  const uint64_t T = qs->target, above1 = qs->above1;
  const float M = key2f(qs->maxkey);
  const int64_t cap = a.dev.ncap[lv];
  const float* sc = a.dev.score[lv] + ((int64_t)kv * GMAX + gi) * cap;
  uint32_t* keep = a.dev.keep[lv] + kv * cap;
  const int32_t* cand = a.dev.cand + (int64_t)hq * a.dev.ncap[1];
  const uint32_t ncand = qs->ncand;
  const uint32_t bit = 1u << gi;
  // fine histogram of the boundary bin's candidates
  for (int i = threadIdx.x; i < NB2; i += 256) h2[i] = 0ull;
  __syncthreads();
  for (uint32_t i = threadIdx.x; i < ncand; i += 256) {
    const BinMass bm = bin_mass(sc[cand[i]], M);
    atomicAdd(&h2[bm.sub], (unsigned long long)bm.mass);
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    uint32_t bb;
    uint64_t ab, dummy;
    wave_boundary512((const uint64_t*)h2, above1, T, threadIdx.x, bb, ab, dummy);
    if (threadIdx.x == 0) { bin = bb; above = ab; ntie = 0; }
  }
  __syncthreads();
  const uint32_t b2 = bin;
  const uint64_t above2 = above;
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

// Children of the kept entries of one chunk, written to consecutive output slots.  The
// union list is in ascending node order, so only the level's last node can have fewer than
// b children and it is the last kept entry wherever it appears: output slot o of the chunk
// is child o % b of the chunk's (o / b)-th kept entry (at level 1: the o-th kept block).
__global__ __launch_bounds__(256) void route_expand_emit_kernel(RouteArgs a) {
  __shared__ int32_t red[4], red2[4], wk[4];
  __shared__ int32_t knode[EXPAND_CHUNK];
  __shared__ uint32_t kmask[EXPAND_CHUNK];
  __shared__ int32_t total_s;
  const int kv = blockIdx.y, lv = a.level;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
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
  if (lane == 0) { red[wave] = pre; red2[wave] = tot; }
  if (threadIdx.x == 0) total_s = 0;
  const int64_t c0 = (int64_t)blockIdx.x * EXPAND_CHUNK;
  int32_t nd[EXPAND_CHUNK / 256];
  uint32_t kb[EXPAND_CHUNK / 256];
#pragma unroll
  for (int r = 0; r < EXPAND_CHUNK / 256; ++r) {
    const int64_t e = c0 + r * 256 + threadIdx.x;
    nd[r] = e < cnt ? a.dev.node[lv][kv * cap + e] : 0;
    kb[r] = e < cnt ? a.dev.keep[lv][kv * cap + e] : 0u;
  }
  __syncthreads();
  int32_t mycount = 0;
  int32_t nk = 0;   // kept entries of the earlier rounds (same value in every thread)
  // stable compaction of the kept entries, 256 entries a round; wk is read only between
  // the round's two barriers, so the next round's writes cannot overtake a read
#pragma unroll
  for (int r = 0; r < EXPAND_CHUNK / 256; ++r) {
    const bool k = kb[r] != 0u;
    const uint64_t ball = __ballot(k);
    if (lane == 0) wk[wave] = __popcll(ball);
    __syncthreads();
    int32_t off = nk;
    for (int w = 0; w < wave; ++w) off += wk[w];
    nk += wk[0] + wk[1] + wk[2] + wk[3];
    if (k) {
      const int32_t pos = off + __popcll(ball & ((1ull << lane) - 1ull));
      knode[pos] = nd[r];
      kmask[pos] = kb[r];
      mycount += emitted(a, nd[r], kb[r]);
    }
    __syncthreads();
  }
  for (int off = 1; off < 64; off <<= 1) mycount += __shfl_xor(mycount, off);
  if (lane == 0) atomicAdd(&total_s, mycount);
  __syncthreads();
  const int32_t base = red[0] + red[1] + red[2] + red[3];
  const int out_lv = lv - 1;
  if (blockIdx.x == 0 && threadIdx.x == 0)
    a.dev.cnt[out_lv * a.hkv + kv] = red2[0] + red2[1] + red2[2] + red2[3];
  const int32_t total = total_s;
  const int64_t ocap = a.dev.ncap[out_lv];
  int32_t* onode = a.dev.node[out_lv] + kv * ocap + base;
  uint32_t* omask = a.dev.mask[out_lv] + kv * ocap + base;
  if (lv == 1) {
    for (int32_t o = threadIdx.x; o < total; o += 256) {
      onode[o] = knode[o];
      omask[o] = kmask[o];
    }
  } else {
    const int32_t b = a.b;
    for (int32_t o = threadIdx.x; o < total; o += 256) {
      const int32_t k = o / b, c = o - k * b;
      onode[o] = knode[k] * b + c;
      omask[o] = kmask[k];
    }
  }
}

// ------------------------------------------------------------------ multi-level selection
// Levels whose node count is at most MLS_MAX, selected top-down in one launch per KV head
// after every node of those levels was scored.  One wave per query head.  Per level:
// max of the head's frontier scores; the node's coarse bin (1/8 score unit) and fine
// sub-bin (1/2048) packed in 16 bits in LDS; a wave-private 256-bin histogram of the
// fixed-point masses; the boundary bin; a 256-sub-bin histogram of that bin; the boundary
// sub-bin; exact rank order inside it.  The masses, the target and the rank rule are those
// of the large-frontier path, so a node is kept here exactly when it would be kept there.
// The frontier of the next level is the children of the kept nodes (a bitmap per head);
// after the last level the kept nodes' children become the union list of the next level
// (or the gather list).
constexpr int MNB = 256;                 // coarse bins per head, 1/8 score unit each
constexpr float M_BPU = 8.f;
constexpr int MNB2 = 256;                // fine sub-bins inside the boundary bin
constexpr int M_TIES = 64;               // boundary sub-bin nodes resolved in LDS
constexpr uint16_t M_ABSENT = 0xffffu;   // not in the head's frontier

__device__ __forceinline__ uint16_t mls_binsub(float score, float mx) {
  const float delta = mx - score;
  const float u = delta * M_BPU;
  const uint32_t bin = u < (float)(MNB - 1) ? (uint32_t)u : (uint32_t)(MNB - 1);
  uint32_t sub = 0;
  if (bin < (uint32_t)(MNB - 1)) {
    const float f = (u - (float)bin) * (float)MNB2;
    sub = f < (float)(MNB2 - 1) ? (uint32_t)f : (uint32_t)(MNB2 - 1);
  }
  return (uint16_t)((bin << 8) | sub);   // never M_ABSENT: bin 255 always has sub 0
}
__device__ __forceinline__ uint64_t mls_mass(float score, float mx) {
  const float delta = mx - score;                         // same expression as bin_mass
  return (uint64_t)(expf(-delta) * MASS_SCALE);
}

// Out-of-line copy for the later passes, so the compiler does not keep every node's mass
// alive in registers from the first pass to the last.
__device__ __noinline__ uint64_t mls_mass_ni(float score, float mx) { return mls_mass(score, mx); }

// First bin (of 256 held 4 per lane) where base + inclusive prefix >= target; one wave.
__device__ void wave_boundary256(const uint64_t* bins, uint64_t base, uint64_t target, int lane, uint32_t& bin,
                                 uint64_t& above, uint64_t& total) {
  uint64_t v[4], loc = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) { v[i] = bins[lane * 4 + i]; loc += v[i]; }
  uint64_t inc = loc;
  for (int off = 1; off < 64; off <<= 1) {
    const uint64_t t = __shfl_up(inc, off);
    if (lane >= off) inc += t;
  }
  total = __shfl(inc, 63);
  uint64_t run = base + inc - loc;
  uint32_t fb = 0xffffffffu;
  uint64_t fa = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (fb == 0xffffffffu && run < target && run + v[i] >= target) { fb = lane * 4 + i; fa = run; }
    run += v[i];
  }
  const uint64_t hit = __ballot(fb != 0xffffffffu);
  const int src = hit ? __ffsll((long long)hit) - 1 : 0;
  bin = __shfl(fb, src);
  above = __shfl(fa, src);
}

__global__ __launch_bounds__(GMAX * 64) void route_mls_kernel(RouteArgs a) {
  constexpr int MPL = (MLS_MAX + 63) / 64;    // nodes per lane (node e = 64 i + lane)
  constexpr int MW64 = MPL;                   // 64-bit bitmap words per head
  __shared__ uint64_t h1[GMAX][MNB];
  __shared__ uint64_t h2[GMAX][MNB2];
  __shared__ uint64_t kbm[2][GMAX][MW64];     // kept nodes per head (this level / above)
  __shared__ uint64_t fbm[GMAX][MW64];        // frontier per head (this level)
  __shared__ int32_t ntie[GMAX];
  __shared__ int32_t tie_e[GMAX][M_TIES];
  __shared__ float tie_s[GMAX][M_TIES];
  __shared__ uint64_t tie_m[GMAX][M_TIES];
  __shared__ uint16_t bsl[GMAX][MPL * 64];    // bin | sub code of each node of the head
  __shared__ int32_t eoff[MLS_MAX + 1];
  __shared__ int32_t wsum[GMAX];
  constexpr int NT = GMAX * 64;
  const int kv = blockIdx.x, lane = threadIdx.x & 63, gi = threadIdx.x >> 6;
  const int g = a.g, b = a.b;
  const bool active = gi < g;
  const bool keep_all = a.top_p >= 1.0f;
  int pb = 0;   // kbm[pb] = kept bitmap of the level above
  for (int lv = a.level; lv >= a.dense_lo; --lv) {
    const int n = (int)a.nl[lv];
    const int64_t cap = a.dev.ncap[lv];
    const bool top = lv == a.level;
    for (int i = lane; i < MW64; i += 64) { kbm[pb ^ 1][gi][i] = 0ull; fbm[gi][i] = 0ull; }
    if (lane == 0) ntie[gi] = 0;
    if (active) {
      const float* S = a.dev.score[lv] + ((int64_t)kv * GMAX + gi) * cap;
      // every score of the level in registers (unconditional loads, issued together)
      float v[MPL];
      const float* Sl = S + lane;   // one base register; node 64i + lane at Sl[64 i]
#pragma unroll
      for (int i = 0; i < MPL; ++i) v[i] = (64 * i + lane < n) ? Sl[64 * i] : -INFINITY;
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < MPL; ++i) {
        const int e = 64 * i + lane;
        bool in = e < n;
        if (!top) {
          const int pn = e / b;
          in = in && ((kbm[pb][gi][pn >> 6] >> (pn & 63)) & 1ull);
        }
        const uint64_t fw = __ballot(in);
        if (lane == 0) fbm[gi][i] = fw;
        if (!in) v[i] = -INFINITY;
        mx = fmaxf(mx, v[i]);
        __builtin_amdgcn_sched_barrier(0);
      }
      for (int off = 1; off < 64; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
      if (mx > -INFINITY) {
        uint32_t b1 = 0, b2 = 0;
        uint64_t T = 0, above2 = 0;
        uint16_t* bs = bsl[gi];
        if (!keep_all) {
#pragma unroll
          for (int i = 0; i < 4; ++i) { h1[gi][lane * 4 + i] = 0ull; h2[gi][lane * 4 + i] = 0ull; }
          wave_sync_lds_r();
        }
        // codes to LDS (computed once), coarse histogram
#pragma unroll
        for (int i = 0; i < MPL; ++i) {
          uint16_t code = M_ABSENT;
          if (v[i] > -INFINITY) {
            code = mls_binsub(v[i], mx);
            if (!keep_all)
              atomicAdd((unsigned long long*)&h1[gi][code >> 8], (unsigned long long)mls_mass(v[i], mx));
          }
          bs[64 * i + lane] = code;
          __builtin_amdgcn_sched_barrier(0);   // keep one node's temporaries live at a time
        }
        wave_sync_lds_r();
        if (!keep_all) {
          uint64_t above1, Z, dummy;
          wave_boundary256(h1[gi], 0, ~0ull, lane, b1, above1, Z);
          const double tt = ceil((double)a.top_p * (double)Z);
          T = tt < 1.0 ? 1ull : (uint64_t)tt;
          if (T > Z) T = Z;
          wave_boundary256(h1[gi], 0, T, lane, b1, above1, dummy);
#pragma unroll
          for (int i = 0; i < MPL; ++i) {
            const uint16_t code = bs[64 * i + lane];
            if (code != M_ABSENT && (uint32_t)(code >> 8) == b1)
              atomicAdd((unsigned long long*)&h2[gi][code & 0xffu], (unsigned long long)mls_mass_ni(v[i], mx));
            __builtin_amdgcn_sched_barrier(0);
          }
          wave_sync_lds_r();
          wave_boundary256(h2[gi], above1, T, lane, b2, above2, dummy);
        }
        // kept bitmap above the boundary sub-bin; collect the boundary sub-bin's nodes
#pragma unroll
        for (int i = 0; i < MPL; ++i) {
          bool kp = false;
          const uint16_t code = bs[64 * i + lane];
          if (code != M_ABSENT) {
            const uint32_t bn = code >> 8, sb = code & 0xffu;
            kp = keep_all || bn < b1 || (bn == b1 && sb < b2);
            if (!kp && bn == b1 && sb == b2) {
              const int k = atomicAdd(&ntie[gi], 1);
              if (k < M_TIES) {
                tie_e[gi][k] = 64 * i + lane; tie_s[gi][k] = v[i]; tie_m[gi][k] = mls_mass_ni(v[i], mx);
              }
            }
          }
          const uint64_t kw = __ballot(kp);
          if (lane == 0) kbm[pb ^ 1][gi][i] = kw;
          __builtin_amdgcn_sched_barrier(0);
        }
        wave_sync_lds_r();
        const int nt = keep_all ? 0 : ntie[gi];
        if (nt <= M_TIES) {
          for (int x = lane; x < nt; x += 64) {
            const uint64_t kx = rank_key(tie_s[gi][x], tie_e[gi][x]);
            uint64_t ab = 0;
            for (int y = 0; y < nt; ++y)
              if (rank_key(tie_s[gi][y], tie_e[gi][y]) < kx) ab += tie_m[gi][y];
            if (above2 + ab < T) {
              const int e = tie_e[gi][x];
              atomicOr((unsigned long long*)&kbm[pb ^ 1][gi][e >> 6], 1ull << (e & 63));
            }
          }
        } else {
          // many nodes in one sub-bin: exact rank order by a pass over the frontier
          for (int x = lane; x < n; x += 64) {
            if (!((fbm[gi][x >> 6] >> (x & 63)) & 1ull)) continue;
            const float sx = S[x];
            const uint16_t cx = mls_binsub(sx, mx);
            if ((uint32_t)(cx >> 8) != b1 || (uint32_t)(cx & 0xffu) != b2) continue;
            const uint64_t kx = rank_key(sx, x);
            uint64_t ab = 0;
            for (int y = 0; y < n; ++y) {
              if (!((fbm[gi][y >> 6] >> (y & 63)) & 1ull)) continue;
              const float sy = S[y];
              if (mls_binsub(sy, mx) == cx && rank_key(sy, y) < kx) ab += mls_mass(sy, mx);
            }
            if (above2 + ab < T) atomicOr((unsigned long long*)&kbm[pb ^ 1][gi][x >> 6], 1ull << (x & 63));
          }
        }
      }
    }
    __syncthreads();
    // trace of this level: every node listed; masks / keep = per-head bits of the node
    for (int i = threadIdx.x; i < n; i += NT) {
      uint32_t um = 0, uk = 0;
      for (int h = 0; h < g; ++h) {
        um |= (uint32_t)((fbm[h][i >> 6] >> (i & 63)) & 1ull) << h;
        uk |= (uint32_t)((kbm[pb ^ 1][h][i >> 6] >> (i & 63)) & 1ull) << h;
      }
      a.dev.node[lv][kv * cap + i] = i;
      a.dev.mask[lv][kv * cap + i] = um;
      a.dev.keep[lv][kv * cap + i] = uk;
    }
    if (threadIdx.x == 0) a.dev.cnt[lv * a.hkv + kv] = n;
    pb ^= 1;
    __syncthreads();
  }
  // children of the last level's kept nodes -> union list of the level below (or gather
  // list): per-node output offsets by a block scan; each thread then writes the children
  // of its nodes (adjacent lanes, adjacent nodes)
  const int lv = a.dense_lo;
  const int n = (int)a.nl[lv];
  const int64_t nbelow = lv > 1 ? a.nl[lv - 1] : 0;
  constexpr int PER = (MLS_MAX + NT - 1) / NT;
  auto kept_mask = [&](int e) -> uint32_t {
    uint32_t uk = 0;
    for (int h = 0; h < g; ++h) uk |= (uint32_t)((kbm[pb][h][e >> 6] >> (e & 63)) & 1ull) << h;
    return uk;
  };
  auto nchild = [&](int e, uint32_t uk) -> int32_t {
    if (!uk) return 0;
    return lv == 1 ? 1 : (int32_t)min((int64_t)b, nbelow - (int64_t)e * b);
  };
  const int e0 = threadIdx.x * PER;
  int32_t mine = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = e0 + i;
    if (e < n) mine += nchild(e, kept_mask(e));
  }
  int32_t inc = mine;
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t t = __shfl_up(inc, off);
    if (lane >= off) inc += t;
  }
  if (lane == 63) wsum[gi] = inc;
  __syncthreads();
  int32_t wbase = 0, total = 0;
  for (int w = 0; w < GMAX; ++w) { if (w < gi) wbase += wsum[w]; total += wsum[w]; }
  int32_t run = wbase + inc - mine;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = e0 + i;
    if (e < n) { eoff[e] = run; run += nchild(e, kept_mask(e)); }
  }
  __syncthreads();
  const int out_lv = lv - 1;
  const int64_t ocap = a.dev.ncap[out_lv];
  int32_t* onode = a.dev.node[out_lv] + kv * ocap;
  uint32_t* omask = a.dev.mask[out_lv] + kv * ocap;
  for (int e = threadIdx.x; e < n; e += NT) {
    const uint32_t uk = kept_mask(e);
    const int32_t c = nchild(e, uk);
    const int32_t o = eoff[e];
    for (int j = 0; j < c; ++j) {
      onode[o + j] = lv == 1 ? e : e * b + j;
      omask[o + j] = uk;
    }
  }
  if (threadIdx.x == 0) a.dev.cnt[out_lv * a.hkv + kv] = total;
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
  RouteArgs b = a;
  b.sel_p = (int32_t)grid_for(a.nlevel, 4096, SEL_P);
  hipLaunchKernelGGL(route_hist_kernel, dim3((unsigned)b.sel_p, (unsigned)a.hkv), dim3(SEL_THREADS), 0, st, b);
  hipLaunchKernelGGL(route_bound_kernel, dim3((unsigned)a.hq), dim3(NB1), 0, st, b);
  hipLaunchKernelGGL(route_classify_kernel, dim3((unsigned)b.sel_p, (unsigned)a.hkv), dim3(SEL_THREADS), 0, st, b);
  hipLaunchKernelGGL(route_resolve_kernel, dim3((unsigned)a.hq), dim3(256), 0, st, b);
  return hipGetLastError();
}

template <int D, int R>
static void launch_dense_score_t(const RouteArgs& a, int nlev, hipStream_t st) {
  constexpr int NPB = 4 * (16 / R) * (R >= 8 ? ZHA_SCORE_UN_WIDE : ZHA_SCORE_UN_NARROW);
  int64_t mx = 0;
  for (int l = a.dense_lo; l <= a.level; ++l) mx = a.nl[l] > mx ? a.nl[l] : mx;
  int64_t x = (mx + NPB - 1) / NPB;
  if (x > ZHA_SCORE_GRID) x = ZHA_SCORE_GRID;
  if (x < 1) x = 1;
  hipLaunchKernelGGL((route_score_kernel<D, R>), dim3((unsigned)x, (unsigned)a.hkv, (unsigned)nlev), dim3(256), 0,
                     st, a);
}

hipError_t launch_route_dense_score(const RouteArgs& a, int D, int R, hipStream_t st) {
  const int nlev = a.level - a.dense_lo + 1;
#define ZHA_CASE(DD, RR) else if (D == DD && R == RR) launch_dense_score_t<DD, RR>(a, nlev, st);
  if (false) {}
  ZHA_CASE(64, 1) ZHA_CASE(64, 2) ZHA_CASE(64, 4) ZHA_CASE(64, 8) ZHA_CASE(64, 16)
  ZHA_CASE(128, 1) ZHA_CASE(128, 2) ZHA_CASE(128, 4) ZHA_CASE(128, 8) ZHA_CASE(128, 16)
  else return hipErrorInvalidValue;
#undef ZHA_CASE
  return hipGetLastError();
}

hipError_t launch_route_mls(const RouteArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(route_mls_kernel, dim3((unsigned)a.hkv), dim3(GMAX * 64), 0, st, a);
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
