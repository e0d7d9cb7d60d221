// Top-p selection of one large level.
//
// Blog "Zyphra Hierarchical Attention", section "Routing through the tree": at each level a
// query keeps the smallest set of frontier nodes that holds a fraction p of the estimated
// attention probability (the softmax of the scores over the frontier); nodes are ranked by
// score, equal scores by node id; the set is complete once the cumulative probability
// reaches p; p >= 1 keeps everything.
//
// Probabilities are fixed-point integers: 2^40 is the probability mass of a node scoring
// the head's max, a node's mass is exp(score - max) in that unit.  Integer sums make every
// decision independent of execution order.  Per level and KV head, four launches:
//   hist      per-workgroup coarse histograms of the masses, binned by (max - score) in
//             1/16 score units, one per head of the group, stored whole (no atomics)
//   bound     per head: sum of the partial histograms, the bin where the cumulative mass
//             reaches ceil(p * Z)
//   classify  nodes above that bin are kept; nodes inside it become candidates, staged per
//             wave in LDS and appended with one atomic per head per workgroup
//   resolve   per head: fine histogram (512 sub-bins) of the candidates, the boundary
//             sub-bin, exact rank order inside it (pairwise in LDS, or radix select on the
//             (score, id) key when many nodes tie)
#include "common.hpp"
#include "kernels.hpp"
#include "route_util.hpp"

namespace zha {

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
      // only the scores of heads whose frontier holds the entry are written and read
#pragma unroll
      for (int gi = 0; gi < GMAX; ++gi) v[u][gi] = ((mk[u] >> gi) & 1u) ? sc[(int64_t)gi * cap + e] : 0.f;
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
  // all partials' loads issued together, summed in a fixed order
  uint64_t v[SEL_P];
#pragma unroll
  for (int p = 0; p < SEL_P; ++p) v[p] = p < a.sel_p ? src[(int64_t)p * GMAX * NB1] : 0ull;
  uint64_t sum = 0;
#pragma unroll
  for (int p = 0; p < SEL_P; ++p) sum += v[p];
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
  if (a.top_p[lv] < 1.0f && Z > 0) {
    const double tt = ceil((double)a.top_p[lv] * (double)Z);
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
      // only the scores of heads whose frontier holds the entry are written and read
#pragma unroll
      for (int gi = 0; gi < GMAX; ++gi) v[u][gi] = ((mk[u] >> gi) & 1u) ? sc[(int64_t)gi * cap + e] : 0.f;
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
            const uint32_t bin = bin_of(v[u][gi], Ms[gi]).bin;
            if (bin < B1[gi]) kb |= 1u << gi;
            else cand = bin == B1[gi];
          }
        }
        const uint64_t ball = __ballot(cand);
        if (ball) {
          if (cand) stage[wave][gi][wcnt[gi] + __popcll(ball & ((1ull << lane) - 1ull))] = (int32_t)e;
          wcnt[gi] += (uint32_t)__popcll(ball);
          if (wcnt[gi] > WAVE_STAGE - 64) {   // spill this wave's batch for the head
            wave_sync_lds();
            uint32_t base = 0;
            if (lane == 0) base = atomicAdd(&a.dev.qs[lv * a.hq + kv * g + gi].ncand, wcnt[gi]);
            base = __shfl(base, 0);
            ZHA_CHECK(a.dev, (int64_t)base + wcnt[gi] <= ccap, CHK_CAND_RANGE);
            int32_t* dst = a.dev.cand + (int64_t)(kv * g + gi) * ccap + base;
            for (uint32_t i = lane; i < wcnt[gi]; i += 64) dst[i] = stage[wave][gi][i];
            wave_sync_lds();
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
    ZHA_CHECK(a.dev, (int64_t)off + wcnt_s[wave][gi] <= ccap, CHK_CAND_RANGE);
    int32_t* dst = a.dev.cand + (int64_t)(kv * g + gi) * ccap + off;
    for (uint32_t i = lane; i < wcnt_s[wave][gi]; i += 64) dst[i] = stage[wave][gi][i];
  }
}

// ------------------------------------------------------------------ resolve
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
    const uint32_t sub = bin_of(s, M).sub;
    if (sub < b2) {
      atomicOr(&keep[e], bit);
    } else if (sub == b2) {
      const uint32_t k = atomicAdd(&ntie, 1u);
      if (k < (uint32_t)CAND_PAIRWISE) { tie_e[k] = e; tie_s[k] = s; tie_m[k] = mass_of(s, M); }
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

// ------------------------------------------------------------------ launchers
hipError_t launch_route_select(const RouteArgs& a, hipStream_t st) {
  RouteArgs b = a;
  b.sel_p = (int32_t)grid_for(a.nlevel, 1024, SEL_P);
  hipLaunchKernelGGL(route_hist_kernel, dim3((unsigned)b.sel_p, (unsigned)a.hkv), dim3(SEL_THREADS), 0, st, b);
  hipLaunchKernelGGL(route_bound_kernel, dim3((unsigned)a.hq), dim3(NB1), 0, st, b);
  hipLaunchKernelGGL(route_classify_kernel, dim3((unsigned)b.sel_p, (unsigned)a.hkv), dim3(SEL_THREADS), 0, st, b);
  hipLaunchKernelGGL(route_resolve_kernel, dim3((unsigned)a.hq), dim3(256), 0, st, b);
  return hipGetLastError();
}

}  // namespace zha
