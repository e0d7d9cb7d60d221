// Multi-level selection of the top levels (the levels with at most MLS_MAX nodes), after
// every node of those levels was scored in one launch.  Same top-p rule and fixed-point
// masses as the large-level path (blog "Zyphra Hierarchical Attention", section "Routing
// through the tree").
#include "common.hpp"
#include "kernels.hpp"
#include "route_util.hpp"

namespace zha {

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
          wave_sync_lds();
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
        wave_sync_lds();
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
          wave_sync_lds();
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
        wave_sync_lds();
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
hipError_t launch_route_mls(const RouteArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(route_mls_kernel, dim3((unsigned)a.hkv), dim3(GMAX * 64), 0, st, a);
  return hipGetLastError();
}

}  // namespace zha
