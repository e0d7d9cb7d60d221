// Top-down selection of the upper levels: every level with at most TD_MAX nodes, after all
// nodes of those levels were scored in one launch.  Same top-p rule and fixed-point masses
// as the large-level path (blog "Zyphra Hierarchical Attention", section "Routing through
// the tree": per level, the smallest frontier set whose estimated probability reaches p,
// ranked by score then node id; the next frontier is the kept nodes' children).
//
// One workgroup per query head walks the levels from the top down.  Per level the head's
// frontier is the children of the nodes it kept one level up (an LDS bitmap); the level's
// scores are read once from global memory into LDS (frontier nodes only; the others read
// as -inf), and the passes that follow run on LDS:
//   max -> coarse mass histogram -> boundary bin -> fine histogram of that bin ->
//   boundary sub-bin -> keep / tie classification -> exact rank order among the ties.
// The head's frontier and kept bitmaps of each level go to global memory; a union kernel
// then writes the group's dense union lists (node = position, mask of heads whose frontier
// holds it, mask of heads that kept it), which the list expansion of the lowest such level
// turns into the union list of the level below.
#include "common.hpp"
#include "kernels.hpp"
#include "route_util.hpp"

namespace zha {

constexpr int TD_THREADS = 512;
constexpr int TD_CAND = 1024;  // boundary-bin nodes listed in LDS (more: found by a rescan)
constexpr int TD_TIES = 256;   // boundary sub-bin nodes resolved pairwise in LDS
constexpr uint32_t TD_NONE = 0xffffffffu;

// One wave: loads 512 bins (8 per lane) and the lane's exclusive prefix; the block total.
__device__ __forceinline__ void td_scan512(const unsigned long long* bins, int lane, uint64_t v[8], uint64_t& excl,
                                           uint64_t& total) {
  uint64_t loc = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) { v[i] = bins[lane * 8 + i]; loc += v[i]; }
  uint64_t inc = loc;
  for (int off = 1; off < 64; off <<= 1) {
    const uint64_t t = __shfl_up(inc, off);
    if (lane >= off) inc += t;
  }
  total = __shfl(inc, 63);
  excl = inc - loc;
}

// First bin where base + inclusive prefix >= target (the scanned bins of td_scan512), and the
// mass before it.
__device__ __forceinline__ void td_find(const uint64_t v[8], uint64_t run, uint64_t target, uint32_t& bin,
                                        uint64_t& above) {
  const int lane = threadIdx.x & 63;
  uint32_t fb = TD_NONE;
  uint64_t fa = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (fb == TD_NONE && run < target && run + v[i] >= target) { fb = lane * 8 + i; fa = run; }
    run += v[i];
  }
  const uint64_t hit = __ballot(fb != TD_NONE);
  const int src = hit ? __ffsll((long long)hit) - 1 : 0;
  bin = __shfl(fb, src);
  above = __shfl(fa, src);
}

__global__ __launch_bounds__(TD_THREADS) void route_topdown_kernel(RouteArgs a) {
  constexpr int NW = TD_THREADS / 64;
  // per node of the level: the score (-inf outside the frontier), then its coarse bin
  // (TD_NONE outside the frontier)
  __shared__ __align__(16) uint32_t Cv[TD_MAX];
  __shared__ uint32_t kb2[2][TD_WORDS];        // kept bitmaps: level above / this level
  __shared__ unsigned long long h[NB1];        // coarse, then fine mass histogram, then radix digits
  __shared__ int32_t cand[TD_CAND];
  __shared__ float cand_s[TD_CAND];
  __shared__ int32_t tie_e[TD_TIES];
  __shared__ float tie_s[TD_TIES];
  __shared__ uint64_t tie_m[TD_TIES];
  __shared__ float redm[NW];
  __shared__ uint32_t s_b1, s_b2, s_ncand, s_ntie;
  __shared__ uint64_t s_T, s_above1, s_above2, s_prefix, s_rabove;
  float* Sv = (float*)Cv;
  const int hq = blockIdx.x, kv = hq / a.g, gi = hq % a.g;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = a.b;
  const int lb = (b & (b - 1)) == 0 ? __ffs(b) - 1 : -1;   // log2(b) when b is a power of two
  int pb = 0;   // kb2[pb] = kept bitmap of the level above
  bool empty = false;
  for (int lv = a.level; lv >= a.dense_lo; --lv) {
    const int n = (int)a.nl[lv];
    const int nw = (n + 31) >> 5;
    const bool top = lv == a.level;
    const int64_t cap = a.dev.ncap[lv];
    const float* S = a.dev.score[lv] + ((int64_t)kv * GMAX + gi) * cap;
    uint32_t* gbits = a.dev.tdbits + (((int64_t)lv * a.hq + hq) * 2) * TD_WORDS;   // [frontier | kept]
    uint32_t* kc = kb2[pb ^ 1];
    const uint32_t* kp = kb2[pb];
    // ---- scores of the frontier into LDS (-inf elsewhere), max; float4 loads, all issued
    // before any is used (score rows are 256-byte aligned, the level's row is read whole)
    float mx = -INFINITY;
    constexpr int U = 8;
    const int n4 = (n + 3) >> 2;
    for (int i00 = tid; i00 < n4; i00 += TD_THREADS * U) {
      float4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = i00 + u * TD_THREADS;
        v[u] = (!empty && i < n4) ? *(const float4*)(S + 4 * i) : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = i00 + u * TD_THREADS;
        if (i >= n4) break;
        float x[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
        bool in4 = true;   // b a power of two >= 4: the four nodes share one parent
        if (!top && lb >= 2) {
          const int pn = (4 * i) >> lb;
          in4 = (kp[pn >> 5] >> (pn & 31)) & 1u;
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int e = 4 * i + k;
          bool in = in4 && e < n;
          if (in && !top && lb < 2) {
            const int pn = lb >= 0 ? (e >> lb) : e / b;
            in = (kp[pn >> 5] >> (pn & 31)) & 1u;
          }
          if (!in) x[k] = -INFINITY;
          mx = fmaxf(mx, x[k]);
        }
        *(float4*)(Sv + 4 * i) = make_float4(x[0], x[1], x[2], x[3]);
      }
    }
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    if (lane == 0) redm[wave] = mx;
    for (int i = tid; i < NB1; i += TD_THREADS) h[i] = 0ull;
    __syncthreads();
    float M = redm[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, redm[w]);
    if (M == -INFINITY) {
      // nothing in the frontier: nothing kept here or below
      empty = true;
      for (int w = tid; w < nw; w += TD_THREADS) { gbits[w] = 0u; gbits[TD_WORDS + w] = 0u; kc[w] = 0u; }
      pb ^= 1;
      __syncthreads();
      continue;
    }
    // ---- coarse histogram of the fixed-point masses; the node's bin replaces its score
    for (int e = tid; e < n; e += TD_THREADS) {
      const float x = Sv[e];
      uint32_t code = TD_NONE;
      if (x != -INFINITY) {
        code = bin_of(x, M).bin;
        atomicAdd(&h[code], (unsigned long long)mass_of(x, M));
      }
      Cv[e] = code;
    }
    __syncthreads();
    if (wave == 0) {
      uint64_t v[8], excl, Z;
      td_scan512(h, lane, v, excl, Z);
      uint32_t b1 = NB1;
      uint64_t T = 0, above1 = 0;
      if (a.top_p[lv] < 1.0f && Z > 0) {
        const double tt = ceil((double)a.top_p[lv] * (double)Z);
        T = tt < 1.0 ? 1ull : (uint64_t)tt;
        if (T > Z) T = Z;
        td_find(v, excl, T, b1, above1);
      }
      if (lane == 0) { s_b1 = b1; s_T = T; s_above1 = above1; s_ncand = 0; s_ntie = 0; }
    }
    __syncthreads();
    const uint32_t b1 = s_b1;
    const uint64_t T = s_T;
    // ---- frontier and kept words, one 32-node word per thread (read in a rotated order so
    // the lanes of a wave hit distinct LDS banks); boundary-bin nodes listed
    for (int w = tid; w < nw; w += TD_THREADS) {
      uint32_t c[32];
#pragma unroll
      for (int k = 0; k < 32; ++k) {   // all 32 loads issued before any is used
        const int e = 32 * w + ((k + lane) & 31);
        c[k] = e < n ? Cv[e] : TD_NONE;
      }
      uint32_t fw = 0u, kw = 0u, cw = 0u;
#pragma unroll
      for (int k = 0; k < 32; ++k) {
        const uint32_t bit = 1u << ((k + lane) & 31);
        if (c[k] != TD_NONE) fw |= bit;
        if (c[k] < b1) kw |= bit;
        if (c[k] == b1) cw |= bit;
      }
      gbits[w] = fw;
      kc[w] = kw;
      while (cw) {   // boundary-bin nodes of this word
        const int idx = __ffs(cw) - 1;
        cw &= cw - 1u;
        const uint32_t j = atomicAdd(&s_ncand, 1u);
        if (j < (uint32_t)TD_CAND) cand[j] = 32 * w + idx;
      }
    }
    for (int i = tid; i < NB2; i += TD_THREADS) h[i] = 0ull;
    __syncthreads();
    if (b1 < (uint32_t)NB1) {
      // ---- the boundary bin: its nodes' scores again (global, recently written), fine bins
      const uint32_t nc = s_ncand;
      const bool listed = nc <= (uint32_t)TD_CAND;
      // f(node, score) for every node of the boundary bin
      auto for_each_cand = [&](auto&& f) {
        if (listed) {
          for (uint32_t i = tid; i < nc; i += TD_THREADS) f(cand[i], cand_s[i]);
        } else {
          for (int e = tid; e < n; e += TD_THREADS)
            if (Cv[e] == b1) f(e, S[e]);
        }
      };
      if (listed)
        for (uint32_t i = tid; i < nc; i += TD_THREADS) cand_s[i] = S[cand[i]];
      __syncthreads();
      for_each_cand([&](int e, float x) {
        atomicAdd(&h[bin_of(x, M).sub], (unsigned long long)mass_of(x, M));
      });
      __syncthreads();
      if (wave == 0) {
        uint64_t v[8], excl, tot;
        td_scan512(h, lane, v, excl, tot);
        uint32_t b2;
        uint64_t above2;
        td_find(v, s_above1 + excl, T, b2, above2);
        if (lane == 0) { s_b2 = b2; s_above2 = above2; }
      }
      __syncthreads();
      const uint32_t b2 = s_b2;
      const uint64_t above2 = s_above2;
      for_each_cand([&](int e, float x) {
        const uint32_t sub = bin_of(x, M).sub;
        if (sub < b2) {
          atomicOr(&kc[e >> 5], 1u << (e & 31));
        } else if (sub == b2) {
          const uint32_t k = atomicAdd(&s_ntie, 1u);
          if (k < (uint32_t)TD_TIES) { tie_e[k] = e; tie_s[k] = x; tie_m[k] = mass_of(x, M); }
        }
      });
      __syncthreads();
      const uint32_t nt = s_ntie;
      if (nt <= (uint32_t)TD_TIES) {
        for (uint32_t x = tid; x < nt; x += TD_THREADS) {
          uint64_t ab = 0;
          const uint64_t kx = rank_key(tie_s[x], tie_e[x]);
          for (uint32_t y = 0; y < nt; ++y)
            if (rank_key(tie_s[y], tie_e[y]) < kx) ab += tie_m[y];
          if (above2 + ab < T) atomicOr(&kc[tie_e[x] >> 5], 1u << (tie_e[x] & 31));
        }
      } else {
        // radix select on the 64-bit rank key of the boundary sub-bin's nodes, 8 bits a pass
        unsigned long long* dh = h;   // the fine histogram is no longer needed
        if (tid == 0) { s_prefix = 0; s_rabove = above2; }
        __syncthreads();
        for (int pass = 0; pass < 8; ++pass) {
          const int shift = 56 - 8 * pass;
          const uint64_t hi = pass == 0 ? 0ull : (~0ull << (shift + 8));
          for (int i = tid; i < 256; i += TD_THREADS) dh[i] = 0ull;
          __syncthreads();
          const uint64_t pf = s_prefix;
          for_each_cand([&](int e, float x) {
            if (bin_of(x, M).sub != b2) return;
            const uint64_t k = rank_key(x, e);
            if ((k & hi) == (pf & hi)) atomicAdd(&dh[(k >> shift) & 255u], (unsigned long long)mass_of(x, M));
          });
          __syncthreads();
          if (tid == 0) {
            uint64_t run = s_rabove;
            for (int d = 0; d < 256; ++d) {
              if (run + dh[d] >= T) { s_prefix = pf | ((uint64_t)d << shift); s_rabove = run; break; }
              run += dh[d];
            }
          }
          __syncthreads();
        }
        const uint64_t kb = s_prefix;
        for_each_cand([&](int e, float x) {
          if (bin_of(x, M).sub == b2 && rank_key(x, e) <= kb) atomicOr(&kc[e >> 5], 1u << (e & 31));
        });
      }
      __syncthreads();
    }
    for (int w = tid; w < nw; w += TD_THREADS) gbits[TD_WORDS + w] = kc[w];
    pb ^= 1;
    __syncthreads();
  }
}

// Dense union lists of the top-down levels: entry e = node e, mask / keep = the heads of the
// group whose frontier holds / who kept node e.  A workgroup takes 2,048 nodes of one level
// and KV head; the group's bitmap words for them go through LDS first.
constexpr int UN_NODES = 2048;
__global__ __launch_bounds__(256) void route_topdown_union_kernel(RouteArgs a) {
  constexpr int W = UN_NODES / 32;
  __shared__ uint32_t fb[GMAX][W], kb[GMAX][W];
  const int kv = blockIdx.y, lv = a.level - (int)blockIdx.z, g = a.g;
  const int64_t n = a.nl[lv];
  const int64_t cap = a.dev.ncap[lv];
  const int64_t e0 = (int64_t)blockIdx.x * UN_NODES;
  if (blockIdx.x == 0 && threadIdx.x == 0) a.dev.cnt[lv * a.hkv + kv] = (int32_t)n;
  if (e0 >= n) return;
  const int64_t w0 = e0 / 32, nw = (n + 31) / 32;
  for (int i = threadIdx.x; i < g * W; i += 256) {
    const int gi = i / W, w = i % W;
    const uint32_t* gb = a.dev.tdbits + (((int64_t)lv * a.hq + kv * g + gi) * 2) * TD_WORDS;
    const bool ok = w0 + w < nw;
    fb[gi][w] = ok ? gb[w0 + w] : 0u;
    kb[gi][w] = ok ? gb[TD_WORDS + w0 + w] : 0u;
  }
  __syncthreads();
  const int64_t e1 = e0 + UN_NODES < n ? e0 + UN_NODES : n;
  for (int64_t e = e0 + threadIdx.x; e < e1; e += 256) {
    const int w = (int)((e - e0) >> 5), bit = (int)(e & 31);
    uint32_t fm = 0, km = 0;
    for (int gi = 0; gi < g; ++gi) {
      fm |= ((fb[gi][w] >> bit) & 1u) << gi;
      km |= ((kb[gi][w] >> bit) & 1u) << gi;
    }
    a.dev.node[lv][kv * cap + e] = (int32_t)e;
    a.dev.mask[lv][kv * cap + e] = fm;
    a.dev.keep[lv][kv * cap + e] = km;
  }
}

hipError_t launch_route_topdown(const RouteArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(route_topdown_kernel, dim3((unsigned)a.hq), dim3(TD_THREADS), 0, st, a);
  const int nlev = a.level - a.dense_lo + 1;
  int64_t mx = 0;
  for (int l = a.dense_lo; l <= a.level; ++l) mx = a.nl[l] > mx ? a.nl[l] : mx;
  hipLaunchKernelGGL(route_topdown_union_kernel, dim3(grid_for(mx, UN_NODES, 1 << 20), (unsigned)a.hkv, (unsigned)nlev),
                     dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace zha
