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
// The head's frontier and kept bitmaps of each level go to global memory.  From them one
// kernel writes the (dense) union list of the level below the lowest such level; another
// writes the dense union lists of the selected levels themselves (node = position, mask of
// heads whose frontier holds it, mask of heads that kept it) when they are needed: for a
// trace, or when the lowest selected level is level 1 (its list expansion then gives the
// gather list).
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
    ZHA_CHECK(a.dev, n <= TD_MAX, CHK_TD_SIZE);
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
          if (in && top && a.tf) in = (gbits[e >> 5] >> (e & 31)) & 1u;   // the given frontier
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

// ------------------------------------------------------------------ every level from the keys
// Top-down selection after route_score_allkeys_kernel scored levels 1..4 and wrote the
// level-4 dot products.  One workgroup per query head.  First the levels above level 4 are
// derived from those (a parent's D_j is its children's D_j weighted by exp(LSE_cj - LSE_j);
// its score max_j (D_j + c_j)): dot products in LDS, scores to their global rows.  Then
// every level from a.level down to a.dense_lo is selected by the same rule and fixed-point
// masses as the other top-down kernel, reading the level's score row from global memory in
// three passes (max, coarse histogram, classification) so that no per-node LDS array bounds
// the level size: level 1 of a deep tree has 65K nodes per head.  In each pass a lane takes
// four consecutive nodes (one float4, loaded only when one of them is in the frontier) of a
// 256-node chunk per wave; the kept words come from eight lanes' nibbles.  A level of more
// than TK_LIST_MIN nodes is passed over by kept parent instead: the level above lists its
// kept nodes in LDS (ascending, uint16), and a thread takes one parent and the float4 of its
// four children, all of them frontier nodes, so no lane works on a node outside the
// frontier.  When the selection reaches level 1, the last workgroup of each KV head to
// finish writes the head's gather list (the union of its query heads' kept blocks), so no
// further launch is needed.

// bit i of the byte x -> bits 4i..4i+3 (a block-4 parent's kept bit -> its children's bits)
__device__ __forceinline__ uint32_t spread4(uint32_t x) {
  x = (x | (x << 12)) & 0x000F000Fu;
  x = (x | (x << 6)) & 0x03030303u;
  x = (x | (x << 3)) & 0x11111111u;
  return x * 0xFu;
}

constexpr int TK_THREADS = 1024;
constexpr int TK_U = 5;   // 256-node chunks per wave and round of a selection pass
constexpr int TK_PL = 16384;        // kept parents listed for the level below
constexpr int TK_LIST_MIN = 16384;  // levels above this many nodes are passed over by parent

// The routed blocks of KV head kv once every query head of its group has its level-1 kept
// words: the union over the group's heads of their kept level-1 nodes, ascending, each with
// the mask of heads that kept it (dev.node[0], dev.mask[0], dev.cnt[0] / dev.ucnt[0]).  Per
// 32-node word the OR of the heads' kept words, a workgroup-wide scan of their popcounts,
// then every set bit written at its rank.  wsum: TK_THREADS / 64 + 1 words of LDS.
__device__ __forceinline__ void gather_list(const RouteArgs& a, int kv, uint32_t* wsum) {
  constexpr int NW = TK_THREADS / 64;
  const int g = a.g;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t n = a.nl[1];
  const int nw = (int)((n + 31) / 32);
  const int64_t cap0 = a.dev.ncap[0];
  int32_t* onode = a.dev.node[0] + kv * cap0;
  uint32_t* omask = a.dev.mask[0] + kv * cap0;
  uint32_t* s_base = wsum + NW;
  if (tid == 0) *s_base = 0u;
  __syncthreads();
  for (int w0 = 0; w0 < nw; w0 += TK_THREADS) {
    const int w = w0 + tid;
    uint32_t kw[GMAX];
    uint32_t un = 0u;
#pragma unroll
    for (int gi = 0; gi < GMAX; ++gi) {
      kw[gi] = (gi < g && w < nw) ? td_kept_words(a, 1, kv * g + gi)[w] : 0u;
      un |= kw[gi];
    }
    const int c = __popc(un);
    int inc = c;
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(inc, off);
      if (lane >= off) inc += t;
    }
    if (lane == 63) wsum[wave] = (uint32_t)inc;
    __syncthreads();
    int before = (int)*s_base;
    for (int v = 0; v < wave; ++v) before += (int)wsum[v];
    int total = 0;
    for (int v = 0; v < NW; ++v) total += (int)wsum[v];
    int pos = before + inc - c;
    while (un) {
      const int bit = __ffs(un) - 1;
      un &= un - 1u;
      uint32_t mk = 0u;
#pragma unroll
      for (int gi = 0; gi < GMAX; ++gi) mk |= ((kw[gi] >> bit) & 1u) << gi;
      ZHA_CHECK(a.dev, pos < cap0, CHK_EXPAND_RANGE);
      onode[pos] = 32 * w + bit;
      omask[pos] = mk;
      ++pos;
    }
    __syncthreads();
    if (tid == 0) *s_base += (uint32_t)total;
    __syncthreads();
  }
  if (tid == 0) {
    a.dev.cnt[kv] = (int32_t)*s_base;
    a.dev.ucnt[kv] = (int32_t)*s_base;
  }
}
__global__ __launch_bounds__(TK_THREADS) void route_topdown_keys_kernel(RouteArgs a) {
  constexpr int NW = TK_THREADS / 64;
  constexpr int KW = AK_N1 / 32;
  __shared__ uint32_t kb2[2][KW];              // kept bitmaps: level above / this level
  __shared__ uint32_t fbw[KW];                 // this level's frontier
  __shared__ __align__(16) float Dup[AK_DUP];  // dot products of the levels above level 4
  __shared__ unsigned long long h[NB1];        // coarse, then fine mass histogram, then radix digits
  __shared__ int32_t cand[TD_CAND];
  __shared__ float cand_s[TD_CAND];
  __shared__ int32_t tie_e[TD_TIES];
  __shared__ float tie_s[TD_TIES];
  __shared__ uint64_t tie_m[TD_TIES];
  __shared__ float redm[NW + 1];
  __shared__ uint32_t s_b1, s_b2, s_ncand, s_ntie;
  // the kept nodes of the level above, ascending, when the level below is large (its frontier
  // is their children, four each: the passes then take one kept parent per lane instead of
  // every node slot); s_np > TK_PL: not listed
  __shared__ uint16_t plist[TK_PL];
  __shared__ uint32_t s_np, s_lbase;
  __shared__ uint64_t s_T, s_above1, s_above2, s_prefix, s_rabove;
  const int hq = blockIdx.x, kv = hq / a.g, gi = hq % a.g;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int R = a.nref;
  if (tid == 0) s_np = TK_PL + 1;

  // ---- levels above level 4: dot products and scores.  Thread i of a pass takes item
  // (node i / R, plane i % R); its R-lane group holds one node, whose score is the group's
  // maximum.  All loads of a pass are issued before any is used (children past the level's
  // end read the last child and weigh nothing).
  if (a.level > AK_LC) {
    const int lr = __ffs(R) - 1;   // R is a power of two
    const int64_t cap4 = a.dev.ncap[AK_LC];
    const float* kd = a.dev.kdots + ((int64_t)kv * cap4 * GMAX + gi) * R;   // node c at kd + c * GMAX * R
    int dpo = 0, dco = 0;
    for (int lv = AK_LC + 1; lv <= a.level; ++lv) {
      const int n = (int)a.nl[lv], nc = (int)a.nl[lv - 1];
      const int64_t capl = a.dev.ncap[lv], capc = a.dev.ncap[lv - 1];
      const float* lsep = a.dev.lse[lv] + kv * capl * R;
      const float* lsec = a.dev.lse[lv - 1] + kv * capc * R;
      const float* cp = a.dev.c[lv] + kv * capl * R;
      float* gs = a.dev.score[lv] + ((int64_t)kv * GMAX + gi) * capl;
      const bool from_kd = lv - 1 == AK_LC;
      const int items = n << lr;
      constexpr int UP = 4;
      for (int i0 = 0; i0 < items; i0 += TK_THREADS * UP) {
        float lp[UP], cv[UP], lc[UP][AK_B], dc[UP][AK_B];
#pragma unroll
        for (int u = 0; u < UP; ++u) {
          int i = i0 + u * TK_THREADS + tid;
          i = i < items ? i : items - 1;
          const int node = i >> lr, j = i & (R - 1);
          lp[u] = lsep[i];
          cv[u] = cp[i];
#pragma unroll
          for (int k = 0; k < AK_B; ++k) {
            int c = node * AK_B + k;
            c = c < nc ? c : nc - 1;
            lc[u][k] = lsec[(c << lr) + j];
            // two loads under a uniform branch (a selected pointer would be a generic load)
            if (from_kd) dc[u][k] = kd[(int64_t)c * GMAX * R + j];
            else dc[u][k] = Dup[dpo + (c << lr) + j];
          }
        }
#pragma unroll
        for (int u = 0; u < UP; ++u) {
          const int i = i0 + u * TK_THREADS + tid;
          const int node = (i < items ? i : items - 1) >> lr;
          float acc = 0.f;
#pragma unroll
          for (int k = 0; k < AK_B; ++k)
            if (node * AK_B + k < nc) acc += expf(lc[u][k] - lp[u]) * dc[u][k];
          float m = acc + cv[u];
          for (int off = 1; off < R; off <<= 1) m = fmaxf(m, __shfl_xor(m, off));
          if (i < items) {
            Dup[dco + i] = acc;
            if ((i & (R - 1)) == 0) gs[node] = m;
          }
        }
      }
      __syncthreads();
      dpo = dco;
      dco += items;
    }
  }

  // ---- the levels top-down
  int pb = 0;   // kb2[pb] = kept bitmap of the level above
  bool empty = false;
  for (int lv = a.level; lv >= a.dense_lo; --lv) {
    const int64_t n = a.nl[lv];
    const int nw = (int)((n + 31) >> 5);
    const bool top = lv == a.level;
    ZHA_CHECK(a.dev, nw <= KW, CHK_TD_SIZE);
    // the level's scores: global rows at every level (those above level 4 were written by the
    // pass above), so that every pass compiles to global loads, never to generic ones that
    // would wait together with the LDS reads of the frontier bits
    const float* S = a.dev.score[lv] + ((int64_t)kv * GMAX + gi) * a.dev.ncap[lv];
    uint32_t* gf = td_front_words(a, lv, hq);
    uint32_t* gk = td_kept_words(a, lv, hq);
    uint32_t* kc = kb2[pb ^ 1];
    const uint32_t* kp = kb2[pb];
    const uint32_t np = s_np;
    const bool lst = !top && !empty && np <= (uint32_t)TK_PL;   // kept parents listed
    // ---- the frontier: every node at the top (or the given frontier), else the children of
    // the kept nodes one level up (list mode: this level's kept words start clear)
    for (int w = tid; w < nw; w += TK_THREADS) {
      uint32_t f;
      if (empty) f = 0u;
      else if (top) f = a.tf ? gf[w] : ~0u;
      else f = spread4((kp[w >> 2] >> (8 * (w & 3))) & 0xffu);
      const int64_t rem = n - 32 * (int64_t)w;
      if (rem < 32) f &= (1u << rem) - 1u;
      fbw[w] = f;
      if (lst) kc[w] = 0u;
    }
    for (int i = tid; i < NB1; i += TK_THREADS) h[i] = 0ull;
    __syncthreads();
    // The passes below give lane l of a wave four consecutive nodes (one float4 of scores) of
    // a 256-node chunk, TK_U chunks per wave and round with their loads issued first.  Rows
    // of scores hold whole float4s: node capacities are multiples of 64, LDS levels 32-aligned.
    // the frontier bits of the lane's four nodes of chunk u
    auto front4 = [&](int64_t e0, int u) -> uint32_t {
      const int64_t e = e0 + (int64_t)u * TK_THREADS * 4 + 4 * lane;
      return e < n ? (fbw[e >> 5] >> (e & 31)) & 0xfu : 0u;
    };
    // a lane loads its four scores only when one of them is in the frontier (the others
    // are never read)
    auto load_chunks = [&](int64_t e0, float4 (&x)[TK_U]) {
#pragma unroll
      for (int u = 0; u < TK_U; ++u) {
        const int64_t e = e0 + (int64_t)u * TK_THREADS * 4 + 4 * lane;
        x[u] = front4(e0, u) ? *(const float4*)(S + e) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    };
    constexpr int64_t ROUND = (int64_t)TK_THREADS * 4 * TK_U;   // nodes per round
    // list mode: thread t takes listed parents t, t + TK_THREADS, ...; the float4 of its four
    // children (all in the frontier; those at or past n are not nodes)
    auto load_listed = [&](int i0, float4 (&x)[TK_U]) {
#pragma unroll
      for (int u = 0; u < TK_U; ++u) {
        const int i = i0 + u * TK_THREADS + tid;
        x[u] = *(const float4*)(S + 4 * (int64_t)plist[i < (int)np ? i : (int)np - 1]);
      }
    };
    // ---- pass 1: the frontier's max score; the frontier words out
    float mx = -INFINITY;
    if (lst) {
      for (int i0 = 0; i0 < (int)np; i0 += TK_THREADS * TK_U) {
        float4 x[TK_U];
        load_listed(i0, x);
#pragma unroll
        for (int u = 0; u < TK_U; ++u) {
          const int i = i0 + u * TK_THREADS + tid;
          if (i >= (int)np) break;
          const int64_t e = 4 * (int64_t)plist[i];
          const float xs[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
#pragma unroll
          for (int k = 0; k < 4; ++k) mx = e + k < n ? fmaxf(mx, xs[k]) : mx;
        }
      }
    } else for (int64_t e0 = 256 * wave; e0 < n; e0 += ROUND) {
      float4 x[TK_U];
      load_chunks(e0, x);
#pragma unroll
      for (int u = 0; u < TK_U; ++u) {
        if (e0 + (int64_t)u * TK_THREADS * 4 >= n) break;
        const uint32_t fu = front4(e0, u);
        mx = (fu & 1u) ? fmaxf(mx, x[u].x) : mx;
        mx = (fu & 2u) ? fmaxf(mx, x[u].y) : mx;
        mx = (fu & 4u) ? fmaxf(mx, x[u].z) : mx;
        mx = (fu & 8u) ? fmaxf(mx, x[u].w) : mx;
      }
    }
    for (int w = tid; w < nw; w += TK_THREADS) gf[w] = fbw[w];
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    if (lane == 0) redm[wave] = mx;
    __syncthreads();
    float M = redm[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, redm[w]);
    if (M == -INFINITY) {
      // nothing in the frontier: nothing kept here or below
      empty = true;
      for (int w = tid; w < nw; w += TK_THREADS) { gf[w] = 0u; gk[w] = 0u; kc[w] = 0u; }
      pb ^= 1;
      __syncthreads();
      continue;
    }
    // ---- pass 2: coarse histogram of the fixed-point masses
    if (lst) {
      for (int i0 = 0; i0 < (int)np; i0 += TK_THREADS * TK_U) {
        float4 x[TK_U];
        load_listed(i0, x);
#pragma unroll
        for (int u = 0; u < TK_U; ++u) {
          const int i = i0 + u * TK_THREADS + tid;
          if (i >= (int)np) break;
          const int64_t e = 4 * (int64_t)plist[i];
          const float xs[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
#pragma unroll
          for (int k = 0; k < 4; ++k)
            if (e + k < n) atomicAdd(&h[bin_of(xs[k], M).bin], (unsigned long long)mass_of(xs[k], M));
        }
      }
    } else for (int64_t e0 = 256 * wave; e0 < n; e0 += ROUND) {
      float4 x[TK_U];
      load_chunks(e0, x);
#pragma unroll
      for (int u = 0; u < TK_U; ++u) {
        if (e0 + (int64_t)u * TK_THREADS * 4 >= n) break;
        const uint32_t fu = front4(e0, u);
        const float xs[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if ((fu >> k) & 1u) atomicAdd(&h[bin_of(xs[k], M).bin], (unsigned long long)mass_of(xs[k], M));
      }
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
    // ---- pass 3: kept words (bins before the boundary bin), the nibbles of eight lanes
    // to a word (list mode: each parent's nibble OR-ed in); the boundary bin's nodes (and
    // scores) listed
    if (lst) {
      for (int i0 = 0; i0 < (int)np; i0 += TK_THREADS * TK_U) {
        float4 x[TK_U];
        load_listed(i0, x);
#pragma unroll
        for (int u = 0; u < TK_U; ++u) {
          const int i = i0 + u * TK_THREADS + tid;
          if (i >= (int)np) break;
          const int64_t e = 4 * (int64_t)plist[i];
          const float xs[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
          uint32_t kn = 0u, cn = 0u;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const uint32_t code = bin_of(xs[k], M).bin;
            const uint32_t in = e + k < n ? 1u : 0u;
            kn |= (in & (code < b1 ? 1u : 0u)) << k;
            cn |= (in & (code == b1 ? 1u : 0u)) << k;
          }
          if (kn) atomicOr(&kc[e >> 5], kn << (e & 31));
          if (cn) {
            uint32_t j = atomicAdd(&s_ncand, (uint32_t)__popc(cn));
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              if (!((cn >> k) & 1u)) continue;
              if (j < (uint32_t)TD_CAND) { cand[j] = (int32_t)(e + k); cand_s[j] = xs[k]; }
              ++j;
            }
          }
        }
      }
    } else for (int64_t e0 = 256 * wave; e0 < n; e0 += ROUND) {
      float4 x[TK_U];
      load_chunks(e0, x);
#pragma unroll
      for (int u = 0; u < TK_U; ++u) {
        if (e0 + (int64_t)u * TK_THREADS * 4 >= n) break;
        const uint32_t fu = front4(e0, u);
        const float xs[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
        uint32_t kn = 0u, cn = 0u;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t code = bin_of(xs[k], M).bin;
          const uint32_t in = (fu >> k) & 1u;
          kn |= (in & (code < b1 ? 1u : 0u)) << k;
          cn |= (in & (code == b1 ? 1u : 0u)) << k;
        }
        const int64_t e = e0 + (int64_t)u * TK_THREADS * 4 + 4 * lane;
        uint32_t word = kn << (4 * (lane & 7));
        word |= __shfl_xor(word, 1);
        word |= __shfl_xor(word, 2);
        word |= __shfl_xor(word, 4);
        if ((lane & 7) == 0 && e < n) kc[e >> 5] = word;
        if (cn) {
          uint32_t j = atomicAdd(&s_ncand, (uint32_t)__popc(cn));
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            if (!((cn >> k) & 1u)) continue;
            if (j < (uint32_t)TD_CAND) { cand[j] = (int32_t)(e + k); cand_s[j] = xs[k]; }
            ++j;
          }
        }
      }
    }
    for (int i = tid; i < NB2; i += TK_THREADS) h[i] = 0ull;
    __syncthreads();
    if (b1 < (uint32_t)NB1) {
      const uint32_t nc = s_ncand;
      const bool listed = nc <= (uint32_t)TD_CAND;
      // f(node, score) for every node of the boundary bin
      auto for_each_cand = [&](auto&& fn) {
        if (listed) {
          for (uint32_t i = tid; i < nc; i += TK_THREADS) fn(cand[i], cand_s[i]);
        } else {
          for (int64_t e = tid; e < n; e += TK_THREADS) {
            if (!((fbw[e >> 5] >> (e & 31)) & 1u)) continue;
            const float x = S[e];
            if (bin_of(x, M).bin == b1) fn((int)e, x);
          }
        }
      };
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
        for (uint32_t x = tid; x < nt; x += TK_THREADS) {
          uint64_t ab = 0;
          const uint64_t kx = rank_key(tie_s[x], tie_e[x]);
          for (uint32_t y = 0; y < nt; ++y)
            if (rank_key(tie_s[y], tie_e[y]) < kx) ab += tie_m[y];
          if (above2 + ab < T) atomicOr(&kc[tie_e[x] >> 5], 1u << (tie_e[x] & 31));
        }
      } else {
        // radix select on the 64-bit rank key of the boundary sub-bin's nodes, 8 bits a pass
        unsigned long long* dh = h;
        if (tid == 0) { s_prefix = 0; s_rabove = above2; }
        __syncthreads();
        for (int pass = 0; pass < 8; ++pass) {
          const int shift = 56 - 8 * pass;
          const uint64_t hi = pass == 0 ? 0ull : (~0ull << (shift + 8));
          for (int i = tid; i < 256; i += TK_THREADS) dh[i] = 0ull;
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
    for (int w = tid; w < nw; w += TK_THREADS) gk[w] = kc[w];
    pb ^= 1;
    __syncthreads();
    // ---- the kept nodes listed for a large level below (ascending: per 32-node word the
    // popcounts scanned across the workgroup, then each set bit written at its rank)
    if (lv - 1 >= a.dense_lo && a.nl[lv - 1] > TK_LIST_MIN) {
      uint32_t* wsum = (uint32_t*)redm;
      if (tid == 0) s_lbase = 0u;
      __syncthreads();
      for (int w0 = 0; w0 < nw; w0 += TK_THREADS) {
        const int w = w0 + tid;
        uint32_t word = w < nw ? kb2[pb][w] : 0u;
        const int c = __popc(word);
        int inc = c;
        for (int off = 1; off < 64; off <<= 1) {
          const int t = __shfl_up(inc, off);
          if (lane >= off) inc += t;
        }
        if (lane == 63) wsum[wave] = (uint32_t)inc;
        __syncthreads();
        int pos = (int)s_lbase, total = 0;
        for (int v = 0; v < NW; ++v) {
          if (v < wave) pos += (int)wsum[v];
          total += (int)wsum[v];
        }
        pos += inc - c;
        while (word) {
          const int bit = __ffs(word) - 1;
          word &= word - 1u;
          if (pos < TK_PL) plist[pos] = (uint16_t)(32 * w + bit);
          ++pos;
        }
        __syncthreads();
        if (tid == 0) s_lbase += (uint32_t)total;
        __syncthreads();
      }
      if (tid == 0) s_np = s_lbase <= (uint32_t)TK_PL ? s_lbase : (uint32_t)TK_PL + 1u;
    } else if (tid == 0) {
      s_np = TK_PL + 1;
    }
    __syncthreads();
  }

  // ---- the gather list of the KV head (a decode that reached level 1), written by the last
  // of its g workgroups to finish: each thread's kept words are made visible device-wide
  // before the workgroup counts itself done, and the last one reads the others' after its
  // count
  if (a.tf || a.dense_lo != 1) return;
  __shared__ uint32_t s_last;
  __threadfence();
  __syncthreads();
  if (tid == 0) s_last = atomicAdd(&a.dev.tick[kv], 1u) == (uint32_t)(a.g - 1) ? 1u : 0u;
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  gather_list(a, kv, (uint32_t*)redm);
}

hipError_t launch_route_topdown_keys(const RouteArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(route_topdown_keys_kernel, dim3((unsigned)a.hq), dim3(TK_THREADS), 0, st, a);
  return hipGetLastError();
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
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    a.dev.cnt[lv * a.hkv + kv] = (int32_t)n;
    a.dev.ucnt[lv * a.hkv + kv] = (int32_t)n;
  }
  if (e0 >= n) return;
  const int64_t w0 = e0 / 32, nw = (n + 31) / 32;
  for (int i = threadIdx.x; i < g * W; i += 256) {
    const int gi = i / W, w = i % W;
    const uint32_t* gb = td_front_words(a, lv, kv * g + gi);
    const bool ok = w0 + w < nw;
    fb[gi][w] = ok ? gb[w0 + w] : 0u;
    kb[gi][w] = ok ? gb[td_stride(a, lv) + w0 + w] : 0u;
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

// One workgroup per KV head: clears the group's frontier words of level a.level, then sets
// the bit of every union-list entry for each head in its mask.
__global__ __launch_bounds__(256) void route_td_seed_kernel(RouteArgs a) {
  const int kv = blockIdx.x, lv = a.level, g = a.g;
  const int64_t n = a.nl[lv], nw = (n + 31) / 32, cap = a.dev.ncap[lv];
  for (int64_t i = threadIdx.x; i < (int64_t)g * nw; i += 256) {
    const int gi = (int)(i / nw);
    td_front_words(a, lv, kv * g + gi)[i % nw] = 0u;
  }
  __syncthreads();
  const int64_t cnt = a.dev.cnt[lv * a.hkv + kv];
  for (int64_t e = threadIdx.x; e < cnt; e += 256) {
    const int32_t node = a.dev.node[lv][kv * cap + e];
    const uint32_t mk = a.dev.mask[lv][kv * cap + e];
    if (node < 0 || node >= n) continue;
    for (int gi = 0; gi < g; ++gi)
      if ((mk >> gi) & 1u)
        atomicOr(&td_front_words(a, lv, kv * g + gi)[node >> 5], 1u << (node & 31));
  }
}

hipError_t launch_route_td_seed(const RouteArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(route_td_seed_kernel, dim3((unsigned)a.hkv), dim3(256), 0, st, a);
  return hipGetLastError();
}

// The union list of level dense_lo - 1, dense: entry c = node c for every node of that level,
// its mask = the heads of the group that kept its parent at level dense_lo (0: no head's
// frontier holds it; the large-level kernels then skip it).  Written straight from the
// top-down kept bitmaps, so no compaction pass sits between the top-down selection and the
// next level's scoring.  ucnt counts the entries some head holds.
constexpr int CL_NODES = 4096;                 // children per workgroup
constexpr int CL_WORDS = CL_NODES / 2 / 32 + 2;   // parent bitmap words they span (b >= 2)
__global__ __launch_bounds__(256) void route_td_children_kernel(RouteArgs a) {
  __shared__ uint32_t kb[GMAX][CL_WORDS];
  __shared__ int32_t red[4];
  const int kv = blockIdx.y, g = a.g, lo = a.dense_lo, lc = lo - 1;
  const int64_t nc = a.nl[lc];
  const int64_t capc = a.dev.ncap[lc];
  const int lb = __ffs(a.b) - 1;               // b is a power of two
  const int64_t c0 = (int64_t)blockIdx.x * CL_NODES;
  if (blockIdx.x == 0 && threadIdx.x == 0) a.dev.cnt[lc * a.hkv + kv] = (int32_t)nc;
  if (c0 >= nc) return;
  const int64_t c1 = c0 + CL_NODES < nc ? c0 + CL_NODES : nc;
  const int64_t w0 = (c0 >> lb) >> 5, w1 = (((c1 - 1) >> lb) >> 5) + 1;
  const int nwd = (int)(w1 - w0);
  for (int i = threadIdx.x; i < g * nwd; i += 256) {
    const int gi = i / nwd, w = i % nwd;
    kb[gi][w] = a.dev.tdbits[(((int64_t)lo * a.hq + kv * g + gi) * 2 + 1) * TD_WORDS + w0 + w];
  }
  __syncthreads();
  int32_t nz = 0;
  int32_t* onode = a.dev.node[lc] + kv * capc;
  uint32_t* omask = a.dev.mask[lc] + kv * capc;
  for (int64_t c = c0 + threadIdx.x; c < c1; c += 256) {
    const int64_t pn = c >> lb;
    const int w = (int)((pn >> 5) - w0), bit = (int)(pn & 31);
    uint32_t km = 0;
    for (int gi = 0; gi < g; ++gi) km |= ((kb[gi][w] >> bit) & 1u) << gi;
    onode[c] = (int32_t)c;
    omask[c] = km;
    nz += km != 0u;
  }
  for (int off = 32; off > 0; off >>= 1) nz += __shfl_xor(nz, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = nz;
  __syncthreads();
  if (threadIdx.x == 0) {
    const int32_t t = red[0] + red[1] + red[2] + red[3];
    if (t) atomicAdd(&a.dev.ucnt[lc * a.hkv + kv], t);
  }
}

hipError_t launch_route_topdown(const RouteArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(route_topdown_kernel, dim3((unsigned)a.hq), dim3(TD_THREADS), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_route_td_lists(const RouteArgs& a, hipStream_t st) {
  const int nlev = a.level - a.dense_lo + 1;
  int64_t mx = 0;
  for (int l = a.dense_lo; l <= a.level; ++l) mx = a.nl[l] > mx ? a.nl[l] : mx;
  hipLaunchKernelGGL(route_topdown_union_kernel, dim3(grid_for(mx, UN_NODES, 1 << 20), (unsigned)a.hkv, (unsigned)nlev),
                     dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_route_td_children(const RouteArgs& a, hipStream_t st) {
  const int64_t nc = a.nl[a.dense_lo - 1];
  hipLaunchKernelGGL(route_td_children_kernel, dim3(grid_for(nc, CL_NODES, 1 << 20), (unsigned)a.hkv), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace zha
