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
#include "qk_tile.hpp"

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

// The same scores for bf16 queries on bf16 MFMA.  Each float32 plane element is split
// exactly into three bfloat16 terms (24 significant bits in all); the query is bfloat16
// already, so every product q_e * t_ie is exact in float32 and q.s accumulates in float32 as
// on the float32 path, at three 16x16x32 MFMAs per 32 elements instead of eight 16x16x4.
// Reuse on both operands: a wave keeps the queries of 64 pairs (four 16-pair MFMA blocks) in
// registers for the whole launch and streams plane tiles past them; a workgroup's four
// waves cover 256 pairs.  Each 16-row tile is read from HBM once per workgroup (two float4
// per thread, four tiles in flight), split once and staged in LDS in the MFMA operand
// layout (double-buffered).  Scores go through LDS so that each pair's row is written in
// 16-node (64-byte) runs: a workgroup takes 16 consecutive nodes at a time.
// Grid: (segment slots, Hkv * pair chunks of 256, levels).
constexpr int SG_NODES = 16;

template <int D, int R>
__global__ __launch_bounds__(256) void prefill_score_seg_kernel(PrefillArgs a) {
  constexpr int NPT = 16 / R;                  // nodes per 16-row tile
  constexpr int TPS = SG_NODES / NPT;          // tiles per segment
  constexpr int NL = D / 32;
  constexpr int EL = D / 4;
  constexpr int RW = D + 8;                    // staged row stride (bf16), 16 bytes of padding
  constexpr int F4 = 16 * D / 4 / 256;         // float4 loads per thread per tile
  static_assert(F4 >= 1, "tile of at least 256 float4");
  __shared__ __align__(16) uint16_t stg[2][3][16 * RW];
  __shared__ float cst[2][16];
  __shared__ float buf[4][64][SG_NODES + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, kg = lane >> 4;
  const int kv = (int)blockIdx.y % a.hkv, chunk = (int)blockIdx.y / a.hkv;
  const int lv = 1 + (int)blockIdx.z;
  const int64_t n = a.nl[lv];
  const int64_t cap = a.dev.ncap[lv];
  const float* S = a.dev.s[lv] + (int64_t)kv * cap * R * D;
  const float* C = a.dev.c[lv] + (int64_t)kv * cap * R;
  const int64_t sst = a.sstride[lv];
  float* out = a.S + a.soff[lv] + (int64_t)kv * a.P * sst;
  const int P = a.P, g = a.g;
  const int p0 = chunk * 256 + wave * 64;      // this wave's first pair
  const int64_t nseg = (n + SG_NODES - 1) / SG_NODES;
  if ((int64_t)blockIdx.x >= nseg || chunk * 256 >= P) return;   // whole workgroup
  const bool active = p0 < P;
  // the wave's 64 queries (bf16, exact), four MFMA blocks
  bf16x8 qa[4][NL];
#pragma unroll
  for (int pb = 0; pb < 4; ++pb) {
    const int p = p0 + pb * 16 + col;
    const bf16_t* qp = (const bf16_t*)a.q + ((int64_t)(p / g) * a.hq + (int64_t)kv * g + p % g) * D + kg * EL;
#pragma unroll
    for (int kk = 0; kk < NL; ++kk) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (p < P) v = *(const uint4*)(qp + kk * 8);
      qa[pb][kk] = __builtin_bit_cast(bf16x8, v);
    }
  }
  // tile loads: thread tid takes float4 number tid + 256 * i of the 16 x D tile; NPF tiles
  // in flight (the HBM latency is several tiles' worth of MFMA work)
  constexpr int NPF = TPS < 4 ? TPS : 4;
  float4 ld[NPF][F4];
  float ldc[NPF];
  // every load is unconditional and its value is not touched until the tile is staged
  // (addresses clamped to the level's last node, nodes past it masked when staging): a load
  // under a branch, or a use of its value, makes the compiler wait for every load in flight,
  // which would drain the prefetch
  auto fetch = [&](int64_t tile, float4 (&dst)[F4], float& dc) {
#pragma unroll
    for (int i = 0; i < F4; ++i) {
      const int f = tid + 256 * i;
      const int r = f / (D / 4);
      const int64_t e = min(tile * NPT + r / R, n - 1);
      dst[i] = *(const float4*)(S + (e * R + r % R) * D + (f % (D / 4)) * 4);
    }
    const int rr = tid & 15;
    dc = C[min(tile * NPT + rr / R, n - 1) * R + rr % R];
  };
  // split a fetched tile into stg[bsel]: x = t1 + t2 + t3 exactly, each t the float with the
  // low 16 bits cleared of what is left (8 significant bits each, 24 in all: a float32's
  // whole significand), so the three are exact bfloat16 values; two elements' halves are
  // packed into one word by a byte permute
  auto stage = [&](const float4 (&src_raw)[F4], float sc_raw, int64_t tile, int bsel) {
    float4 src[F4];
#pragma unroll
    for (int i = 0; i < F4; ++i) {
      const int r = (tid + 256 * i) / (D / 4);
      src[i] = tile * NPT + r / R < n ? src_raw[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const float sc = tile * NPT + (tid & 15) / R < n ? sc_raw : -INFINITY;
#pragma unroll
    for (int i = 0; i < F4; ++i) {
      const int f = tid + 256 * i;
      const int r = f / (D / 4), c4 = (f % (D / 4)) * 4;
      const float x[4] = {src[i].x, src[i].y, src[i].z, src[i].w};
      uint32_t t[3][4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t u1 = __float_as_uint(x[u]);
        const float r1 = x[u] - __uint_as_float(u1 & 0xffff0000u);
        const uint32_t u2 = __float_as_uint(r1);
        const float r2 = r1 - __uint_as_float(u2 & 0xffff0000u);
        t[0][u] = u1;
        t[1][u] = u2;
        t[2][u] = __float_as_uint(r2);
      }
#pragma unroll
      for (int sp = 0; sp < 3; ++sp)   // high halves: (t[u] >> 16) | (t[u + 1] & 0xffff0000)
        *(uint2*)&stg[bsel][sp][r * RW + c4] =
            make_uint2(__builtin_amdgcn_perm(t[sp][1], t[sp][0], 0x07060302u),
                       __builtin_amdgcn_perm(t[sp][3], t[sp][2], 0x07060302u));
    }
    if (tid < 16) cst[bsel][tid] = sc;
  };
  float* B = &buf[wave][0][0];
  // this workgroup's tiles in order: segments blockIdx.x, blockIdx.x + gridDim.x, ...
  const int64_t nmine = (nseg - (int64_t)blockIdx.x + gridDim.x - 1) / gridDim.x;
  const int64_t Q = nmine * TPS;
  auto tile_of = [&](int64_t q) { return ((int64_t)blockIdx.x + (q / TPS) * gridDim.x) * TPS + q % TPS; };
  const int64_t last_tile = tile_of(Q - 1);
  auto tile_at = [&](int64_t q) { return q < Q ? tile_of(q) : last_tile; };
#pragma unroll
  for (int j = 0; j < NPF; ++j) fetch(tile_at(j), ld[j], ldc[j]);
  stage(ld[0], ldc[0], tile_at(0), 0);
  __syncthreads();
  // the scores of tile q are finished (plane max, LDS buffer) while tile q + 1's MFMAs run
  auto finish = [&](const f32x4 (&acc)[4], const float (&cr)[4], int64_t q) {
    const int tt = (int)(q % TPS);
#pragma unroll
    for (int pb = 0; pb < 4; ++pb) {
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = a.sigma * acc[pb][e] + cr[e];
      // row 4kg+e is plane (4kg+e) % R of node (4kg+e) / R: the max over a node's planes
      // within the lane's four rows, then across lane groups for R > 4
      float* dst = B + (pb * 16 + col) * (SG_NODES + 1) + tt * NPT;
      if constexpr (R == 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[4 * kg + e] = v[e];
      } else if constexpr (R == 2) {
        dst[2 * kg] = fmaxf(v[0], v[1]);
        dst[2 * kg + 1] = fmaxf(v[2], v[3]);
      } else {
        float m = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
        if constexpr (R >= 8) m = fmaxf(m, __shfl_xor(m, 16));
        if constexpr (R >= 16) m = fmaxf(m, __shfl_xor(m, 32));
        if ((kg & (R / 4 - 1)) == 0) dst[(4 * kg) / R] = m;
      }
    }
    if (tt == TPS - 1) {
      // the wave's 64 rows of this segment (the buffer is the wave's own)
      wave_sync_lds();
      const int64_t node0 = ((int64_t)blockIdx.x + (q / TPS) * gridDim.x) * SG_NODES;
      const int64_t nn = min((int64_t)SG_NODES, n - node0);
      constexpr int RPI = 64 / SG_NODES;       // rows per store instruction
#pragma unroll 4
      for (int r = 0; r < 64; r += RPI) {
        const int pr = r + lane / SG_NODES, jn = lane % SG_NODES;
        const int p = p0 + pr;
        if (p < P && jn < nn) out[(int64_t)p * sst + node0 + jn] = B[pr * (SG_NODES + 1) + jn];
      }
      wave_sync_lds();
    }
  };
  f32x4 accp[4];
  float crp[4];
  int cur = 0;
  for (int64_t q0 = 0; q0 < Q; q0 += NPF) {
#pragma unroll
    for (int j = 0; j < NPF; ++j) {
      const int64_t q = q0 + j;
      fetch(tile_at(q + NPF), ld[j], ldc[j]);   // tile q was staged already
      f32x4 acc[4];
      float cr[4];
      if (active) {
        bf16x8 s1[NL], s2[NL], s3[NL];
#pragma unroll
        for (int kk = 0; kk < NL; ++kk) {
          const int off = col * RW + kg * EL + kk * 8;
          s1[kk] = __builtin_bit_cast(bf16x8, *(const uint4*)&stg[cur][0][off]);
          s2[kk] = __builtin_bit_cast(bf16x8, *(const uint4*)&stg[cur][1][off]);
          s3[kk] = __builtin_bit_cast(bf16x8, *(const uint4*)&stg[cur][2][off]);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) cr[e] = cst[cur][4 * kg + e];
        // plane rows x pairs: lane (kg, col) gets rows 4kg..4kg+3 of pair col; four
        // independent accumulation chains (one per 16-pair block), smallest terms first
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) acc[pb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < NL; ++kk) {
#pragma unroll
          for (int pb = 0; pb < 4; ++pb) acc[pb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(s3[kk], qa[pb][kk], acc[pb], 0, 0, 0);
#pragma unroll
          for (int pb = 0; pb < 4; ++pb) acc[pb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(s2[kk], qa[pb][kk], acc[pb], 0, 0, 0);
#pragma unroll
          for (int pb = 0; pb < 4; ++pb) acc[pb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(s1[kk], qa[pb][kk], acc[pb], 0, 0, 0);
        }
        if (q > 0) finish(accp, crp, q - 1);
      }
      if (q + 1 < Q) stage(ld[(j + 1) % NPF], ldc[(j + 1) % NPF], tile_of(q + 1), cur ^ 1);
      __syncthreads();
      cur ^= 1;
#pragma unroll
      for (int pb = 0; pb < 4; ++pb) accp[pb] = acc[pb];
#pragma unroll
      for (int e = 0; e < 4; ++e) crp[e] = cr[e];
    }
  }
  if (active) finish(accp, crp, Q - 1);
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
constexpr int PS_LIST = 6144;   // frontier nodes held in LDS (more: the level is read from global memory)
constexpr int PS_TIES = 256;    // boundary sub-bin nodes resolved pairwise (more: radix select)
constexpr int PS_KWORDS = 2048; // kept bitmap words built in LDS (a longer level: in global memory)

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
// is held in one of three ways for the passes that follow:
//   list    at most PS_LIST nodes: node ids and scores in LDS;
//   sparse  a longer frontier covering under a quarter of its level: every pass walks the
//           parents' kept bitmap (in LDS when it fits) and reads the kept parents' children;
//   scan    a denser frontier: every pass reads the whole level from global memory
//           (PS_UNROLL loads in flight per thread), the frontier test from that bitmap.
// Nodes outside the pair's tree score -inf and drop out.
constexpr int PS_UNROLL = 8;

__global__ __launch_bounds__(PS_THREADS, 4) void prefill_select_kernel(PrefillArgs a) {
  constexpr int NW = PS_THREADS / 64;
  __shared__ uint32_t lbuf[2 * PS_LIST];   // the list (ids, scores), or the parents' kept bitmap
  int32_t* fl = (int32_t*)lbuf;
  float* fs = (float*)(lbuf + PS_LIST);
  __shared__ unsigned long long h[NB1];
  __shared__ int32_t tie_e[PS_TIES];
  __shared__ float tie_s[PS_TIES];
  __shared__ uint64_t tie_m[PS_TIES];
  __shared__ float redm[NW];
  __shared__ int32_t wsum[NW];
  __shared__ uint32_t kl[PS_KWORDS];
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
    const bool lds_kept = nw <= PS_KWORDS;
    // ---- the frontier
    int64_t nf = 0;
    const int64_t nwp = top ? 0 : (a.nl[lv + 1] + 31) >> 5;   // parent bitmap words
    if (top) {
      nf = n;
      if (n <= PS_LIST)
        for (int k = tid; k < (int)n; k += PS_THREADS) { fl[k] = k; fs[k] = row[k]; }
    } else {
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
            for (int64_t e = first; e < last; ++e, ++off) fl[off] = (int32_t)e;
          }
        }
        nf += round;
      }
      // the listed nodes' scores, all threads at once
      if (nf <= PS_LIST) {
        __syncthreads();
        for (int64_t k = tid; k < nf; k += PS_THREADS) fs[k] = row[fl[k]];
      }
    }
    const bool list = nf <= PS_LIST;
    const bool sparse = !list && !top && nf * 4 < n;
    // past the list: the parents' kept bitmap goes to LDS (in the list's space) when it fits
    uint32_t* pbits = lbuf;
    const bool lds_bits = !list && !top && nwp <= 2 * PS_LIST;
    __syncthreads();
    if (lds_bits)
      for (int64_t w = tid; w < nwp; w += PS_THREADS) pbits[w] = ld_agent(kp + w);
    // kept marks: LDS bitmap (copied out at the end) or the global one; a listed or sparse
    // frontier sets bits a node or a parent at a time, so its bitmap starts cleared (a
    // scanned level writes every word in its classification pass)
    if (list || sparse) {
      if (lds_kept)
        for (int64_t w = tid; w < nw; w += PS_THREADS) kl[w] = 0u;
      else
        for (int64_t w = tid; w < nw; w += PS_THREADS) kb[w] = 0u;
    }
    __syncthreads();
    auto in_front = [&](int64_t k) -> bool {
      if (top) return true;
      const int64_t pn = k >> lb;
      return ((lds_bits ? pbits[pn >> 5] : ld_agent(kp + (pn >> 5))) >> (pn & 31)) & 1u;
    };
    auto pword = [&](int64_t w) -> uint32_t { return lds_bits ? pbits[w] : ld_agent(kp + w); };
    // f(node, score) for every entry (score -inf outside the frontier)
    auto each = [&](auto&& f) {
      if (list) {
        for (int64_t k = tid; k < nf; k += PS_THREADS) f((int64_t)fl[k], fs[k]);
      } else if (sparse) {
        for (int64_t w = tid; w < nwp; w += PS_THREADS)
          for (uint32_t r = pword(w); r; r &= r - 1u) {
            const int64_t first = (32 * w + __ffs(r) - 1) << lb;
            const int64_t last = min(first + b, n);
            for (int64_t e = first; e < last; ++e) f(e, row[e]);
          }
      } else {
        for (int64_t k0 = tid; k0 < n; k0 += (int64_t)PS_UNROLL * PS_THREADS) {
          float xs[PS_UNROLL];
#pragma unroll
          for (int j = 0; j < PS_UNROLL; ++j) {
            const int64_t k = k0 + (int64_t)j * PS_THREADS;
            xs[j] = (k < n && in_front(k)) ? row[k] : -INFINITY;
          }
#pragma unroll
          for (int j = 0; j < PS_UNROLL; ++j) f(k0 + (int64_t)j * PS_THREADS, xs[j]);
        }
      }
    };
    auto keep = [&](int64_t e) {
      if (lds_kept) atomicOr(&kl[e >> 5], 1u << (e & 31));
      else atomicOr(&kb[e >> 5], 1u << (e & 31));
    };
    // ---- max
    float mx = -INFINITY;
    each([&](int64_t, float x) { mx = fmaxf(mx, x); });
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    if (lane == 0) redm[wave] = mx;
    for (int k = tid; k < NB1; k += PS_THREADS) h[k] = 0ull;
    __syncthreads();
    float M = redm[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, redm[w]);
    if (M == -INFINITY) {   // empty frontier: nothing kept here or below
      for (int64_t w = tid; w < nw; w += PS_THREADS) kb[w] = 0u;
      __syncthreads();
      continue;
    }
    // ---- coarse histogram of the fixed-point masses
    each([&](int64_t, float x) {
      if (x != -INFINITY) atomicAdd(&h[bin_of(x, M).bin], (unsigned long long)mass_of(x, M));
    });
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
    if (list) {
      each([&](int64_t e, float x) {
        if (x == -INFINITY) return;
        const BinSub bs = bin_of(x, M);
        if (bs.bin < b1) keep(e);
        else if (bs.bin == b1) atomicAdd(&h[bs.sub], (unsigned long long)mass_of(x, M));
      });
    } else if (sparse) {
      // a kept parent's children share bitmap words with no other parent's (b a power of
      // two): their kept bits go in with one atomic per word
      uint32_t* kw = lds_kept ? kl : kb;
      for (int64_t w = tid; w < nwp; w += PS_THREADS)
        for (uint32_t r = pword(w); r; r &= r - 1u) {
          const int64_t first = (32 * w + __ffs(r) - 1) << lb;
          const int64_t last = min(first + b, n);
          uint32_t m = 0u;
          for (int64_t e = first; e < last; ++e) {
            const float x = row[e];
            if (x != -INFINITY) {
              const BinSub bs = bin_of(x, M);
              if (bs.bin < b1) m |= 1u << (e & 31);
              else if (bs.bin == b1) atomicAdd(&h[bs.sub], (unsigned long long)mass_of(x, M));
            }
            if ((e & 31) == 31 || e + 1 == last) {
              if (m) {
                if (b >= 32) kw[e >> 5] = m;   // a whole word of this parent's
                else atomicOr(&kw[e >> 5], m);
              }
              m = 0u;
            }
          }
        }
    } else {
      // each wave's 64 consecutive nodes of a round give two kept words by one ballot
      for (int64_t k0 = tid; k0 - lane < n; k0 += (int64_t)PS_UNROLL * PS_THREADS) {
        float xs[PS_UNROLL];
#pragma unroll
        for (int j = 0; j < PS_UNROLL; ++j) {
          const int64_t k = k0 + (int64_t)j * PS_THREADS;
          xs[j] = (k < n && in_front(k)) ? row[k] : -INFINITY;
        }
#pragma unroll
        for (int j = 0; j < PS_UNROLL; ++j) {
          const float x = xs[j];
          bool kept = false;
          if (x != -INFINITY) {
            const BinSub bs = bin_of(x, M);
            kept = bs.bin < b1;
            if (bs.bin == b1) atomicAdd(&h[bs.sub], (unsigned long long)mass_of(x, M));
          }
          const uint64_t m = __ballot(kept);
          const int64_t w0 = (k0 - lane + (int64_t)j * PS_THREADS) >> 5;
          if (lane < 2 && w0 + lane < nw) {
            const uint32_t word = lane ? (uint32_t)(m >> 32) : (uint32_t)m;
            if (lds_kept) kl[w0 + lane] = word;
            else kb[w0 + lane] = word;
          }
        }
      }
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
      each([&](int64_t e, float x) {
        if (x == -INFINITY) return;
        const BinSub bs = bin_of(x, M);
        if (bs.bin != b1) return;
        if (bs.sub < b2) {
          keep(e);
        } else if (bs.sub == b2) {
          const uint32_t j = atomicAdd(&s_ntie, 1u);
          if (j < (uint32_t)PS_TIES) { tie_e[j] = (int32_t)e; tie_s[j] = x; tie_m[j] = mass_of(x, M); }
        }
      });
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
          if (above2 + ab < T) keep(tie_e[x]);
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
          each([&](int64_t e, float x) {
            if (x == -INFINITY) return;
            const BinSub bs = bin_of(x, M);
            if (bs.bin != b1 || bs.sub != b2) return;
            const uint64_t rk = rank_key(x, (int32_t)e);
            if ((rk & hi) == (pf & hi)) atomicAdd(&dh[(rk >> shift) & 255u], (unsigned long long)mass_of(x, M));
          });
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
        each([&](int64_t e, float x) {
          if (x == -INFINITY) return;
          const BinSub bs = bin_of(x, M);
          if (bs.bin == b1 && bs.sub == b2 && rank_key(x, (int32_t)e) <= kbnd) keep(e);
        });
      }
    }
    __syncthreads();
    if (lds_kept) {
      for (int64_t w = tid; w < nw; w += PS_THREADS) kb[w] = kl[w];
      __syncthreads();
    }
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

// ---------------------------------------------------------------- union attention
// The routed attention of a whole sub-batch on bf16 MFMA.  The queries of a sub-batch
// keep overlapping block sets (on deep each head keeps about a quarter of the blocks and
// their union is nearly all of them), so instead of one gather list per query the K/V
// tiles are read once for all pairs: a workgroup takes a run of level-1 bitmap words
// (32 blocks each) of one KV head and 128 pairs (a wave 32 of them, two MFMA blocks);
// per word the wave ORs its pairs' kept words and skips the word, a 32-token tile, or a
// 16-pair block's work on a tile, when none of those pairs keeps a block there; per tile
// S^T = K.Q^T (tokens x pairs), each pair
// masked to its own kept blocks, its tokens up to its position and the sink, an online
// softmax per pair, and P.V with the V tile transposed through LDS (the dense MFMA
// attention's scheme, with pairs in place of heads).  Partials (max, sum, o) per pair and
// split are merged by prefill_combine_kernel.
constexpr int PA_NPB = 2;        // 16-pair MFMA blocks per wave
constexpr int PA_CHUNK = 4 * 16 * PA_NPB;   // pairs per workgroup
constexpr int PA_WGS = 512;      // workgroups of one launch (two per compute unit)
constexpr int PA_SPLITS = 128;   // splits per (KV head, pair chunk), at most
constexpr int PA_VS = 36;        // LDS row stride of the transposed V tile (bf16)

template <int D>
__global__ __launch_bounds__(256, 2) void prefill_attend_kernel(PrefillArgs a, float* part, int nsplit) {
  constexpr int NK = D / 32;      // 8-element groups per lane of a K row or a query
  constexpr int NM = D / 16;      // output dim blocks
  __shared__ __align__(16) uint16_t vt_all[4][D * PA_VS];
  __shared__ float al_all[4][PA_NPB][16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, kg = lane >> 4;
  const int kv = (int)blockIdx.y % a.hkv, chunk = (int)blockIdx.y / a.hkv, split = blockIdx.x;
  const int P = a.P, g = a.g, lb = __ffs(a.b) - 1;
  const int p0 = chunk * PA_CHUNK + wave * 16 * PA_NPB;
  if (p0 >= P) return;                        // a whole wave; no workgroup barriers below
  const int64_t nend = a.N0 + a.mb;          // tokens in the tree
  const int64_t nw = (a.nl[1] + 31) >> 5;
  const int64_t wper = (nw + nsplit - 1) / nsplit;
  const int64_t w0 = (int64_t)split * wper, w1 = min(nw, w0 + wper);
  const bf16_t* Kb = (const bf16_t*)a.K + (int64_t)kv * a.cap * D;
  const bf16_t* Vb = (const bf16_t*)a.V + (int64_t)kv * a.cap * D;
  uint16_t* Vt = vt_all[wave];
  // the queries of the wave's 16-pair blocks (B operand: pair col, 8 elements per group)
  bf16x8 qf[PA_NPB][NK];
  int64_t posc[PA_NPB];                       // position of pair col of each block
#pragma unroll
  for (int pb = 0; pb < PA_NPB; ++pb) {
    const int p = p0 + pb * 16 + col;
    posc[pb] = p < P ? a.N0 + p / g : -1;
    const bf16_t* qp = (const bf16_t*)a.q + ((int64_t)(p / g) * a.hq + (int64_t)kv * g + p % g) * D + kg * (D / 4);
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (p < P) v = *(const uint4*)(qp + kk * 8);
      qf[pb][kk] = __builtin_bit_cast(bf16x8, v);
    }
  }
  // lane j < 16 * PA_NPB reads the kept words of pair p0 + j
  const bool lane_pair = lane < 16 * PA_NPB && p0 + lane < P;
  const uint32_t* kbp = a.KB + a.koff[1] + ((int64_t)kv * a.P + p0 + (lane_pair ? lane : 0)) * a.kstride[1];
  float m[PA_NPB], l[PA_NPB];
  f32x4 acc[PA_NPB][NM];
#pragma unroll
  for (int pb = 0; pb < PA_NPB; ++pb) {
    m[pb] = -INFINITY;
    l[pb] = 0.f;
#pragma unroll
    for (int i = 0; i < NM; ++i) acc[pb][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int vtk = lane & 31, vc = lane >> 5;  // V loads: token vtk, dims 16i + 8vc .. +7
  for (int64_t w = w0; w < w1; ++w) {
    const uint32_t kw = lane_pair ? kbp[w] : 0u;
    uint32_t kc[PA_NPB], ab[PA_NPB];          // kept word of pair col of each block; the block's OR
    uint32_t any = 0u;
#pragma unroll
    for (int pb = 0; pb < PA_NPB; ++pb) {
      kc[pb] = __shfl(kw, pb * 16 + col);
      uint32_t o = kc[pb];
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) o |= __shfl_xor(o, off);
      if (a.keep_sink && w == 0) o |= 1u;     // the sink's block
      ab[pb] = o;
      any |= o;
    }
    if (!any) continue;
    const int64_t tb = (w * 32) << lb;
    const int64_t te = min(((w + 1) * 32) << lb, nend);
    for (int64_t t0 = tb; t0 < te; t0 += 32) {
      const int e0 = (int)((t0 >> lb) & 31);
      const uint32_t span = lb >= 5 ? 1u : (1u << (32 >> lb)) - 1u;   // blocks of the tile
      if (!((any >> e0) & span)) continue;
      uint4 kf[2][NK];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int64_t tk = t0 + st * 16 + col;
        if (tk < nend) Qk<bf16_t, D>::load_k(Kb + tk * D, kg, kf[st]);
        else
#pragma unroll
          for (int kk = 0; kk < NK; ++kk) kf[st][kk] = make_uint4(0, 0, 0, 0);
      }
      uint4 vv[NM];
      {
        const int64_t tk = t0 + vtk;
#pragma unroll
        for (int i = 0; i < NM; ++i)
          vv[i] = tk < nend ? *(const uint4*)(Vb + tk * D + 16 * i + 8 * vc) : make_uint4(0, 0, 0, 0);
      }
      uint32_t pbits[PA_NPB][4];              // P rows of pair col of each block, bf16 pairs
      bool act[PA_NPB];                       // blocks with a pair keeping a block of the tile
#pragma unroll
      for (int pb = 0; pb < PA_NPB; ++pb) {
        act[pb] = (ab[pb] >> e0) & span;
        if (!act[pb]) continue;
        float sc[2][4];
        float rmax = -INFINITY;
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          f32x4 s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < NK; ++kk)
            s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf[st][kk]), qf[pb][kk], s4, 0, 0, 0);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int64_t tok = t0 + st * 16 + kg * 4 + e;
            const bool kept = (kc[pb] >> ((tok >> lb) & 31)) & 1u;
            const bool use = tok <= posc[pb] && (kept || (a.keep_sink && tok == 0));
            sc[st][e] = use ? a.sigma * s4[e] : -INFINITY;
            rmax = fmaxf(rmax, sc[st][e]);
          }
        }
        rmax = fmaxf(rmax, __shfl_xor(rmax, 16));
        rmax = fmaxf(rmax, __shfl_xor(rmax, 32));
        const float mn = fmaxf(m[pb], rmax);
        const float alpha = mn == -INFINITY ? 1.f : expf(m[pb] - mn);
        float rsum = 0.f;
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int e = 0; e < 4; e += 2) {
            const float q0 = mn == -INFINITY ? 0.f : expf(sc[st][e] - mn);
            const float q1 = mn == -INFINITY ? 0.f : expf(sc[st][e + 1] - mn);
            rsum += q0 + q1;
            pbits[pb][st * 2 + e / 2] = f2bf16_bits(q0) | (f2bf16_bits(q1) << 16);
          }
        rsum += __shfl_xor(rsum, 16);
        rsum += __shfl_xor(rsum, 32);
        l[pb] = l[pb] * alpha + rsum;
        m[pb] = mn;
        if (kg == 0) al_all[wave][pb][col] = alpha;
      }
      // the V tile, transposed: Vt[dim][token]
#pragma unroll
      for (int i = 0; i < NM; ++i) {
        const uint32_t w4[4] = {vv[i].x, vv[i].y, vv[i].z, vv[i].w};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int d = 16 * i + 8 * vc + k;
          Vt[d * PA_VS + vtk] = (uint16_t)((w4[k >> 1] >> (16 * (k & 1))) & 0xffffu);
        }
      }
      wave_sync_lds();
#pragma unroll
      for (int pb = 0; pb < PA_NPB; ++pb) {
        if (!act[pb]) continue;
        float ah[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) ah[e] = al_all[wave][pb][4 * kg + e];
        const bf16x8 pa = __builtin_bit_cast(bf16x8, make_uint4(pbits[pb][0], pbits[pb][1], pbits[pb][2], pbits[pb][3]));
#pragma unroll
        for (int i = 0; i < NM; ++i) {
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[pb][i][e] *= ah[e];
          const uint16_t* vrow = Vt + (16 * i + col) * PA_VS;
          const uint2 lo = *(const uint2*)(vrow + 4 * kg);
          const uint2 hi = *(const uint2*)(vrow + 16 + 4 * kg);
          const bf16x8 vb = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
          acc[pb][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb, acc[pb][i], 0, 0, 0);
        }
      }
      wave_sync_lds();
    }
  }
  // partials [Hkv][P][nsplit][D + 2]: acc[pb][i][e] = pair pb*16 + 4kg + e, dim 16i + col
#pragma unroll
  for (int pb = 0; pb < PA_NPB; ++pb) {
    const int pc = p0 + pb * 16 + col;
    if (kg == 0 && pc < P) {
      float* pp = part + (((int64_t)kv * P + pc) * nsplit + split) * (D + 2);
      pp[0] = m[pb];
      pp[1] = l[pb];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int pr = p0 + pb * 16 + 4 * kg + e;
      if (pr < P) {
        float* pp = part + (((int64_t)kv * P + pr) * nsplit + split) * (D + 2) + 2;
#pragma unroll
        for (int i = 0; i < NM; ++i) pp[16 * i + col] = acc[pb][i][e];
      }
    }
  }
}

// Per pair: the splits merged (max-rescaled sums), o = sum / normaliser, written to the
// query's output row.  Grid (P, Hkv), D threads.
template <int D>
__global__ __launch_bounds__(D) void prefill_combine_kernel(PrefillArgs a, const float* part, int nsplit, float* out) {
  const int p = blockIdx.x, kv = blockIdx.y, d = threadIdx.x;
  const float* pp = part + ((int64_t)kv * a.P + p) * nsplit * (D + 2);
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, pp[(int64_t)s * (D + 2)]);
  float L = 0.f, O = 0.f;
  if (M > -INFINITY)
    for (int s = 0; s < nsplit; ++s) {
      const float ms = pp[(int64_t)s * (D + 2)];
      if (ms == -INFINITY) continue;
      const float w = expf(ms - M);
      L += pp[(int64_t)s * (D + 2) + 1] * w;
      O += pp[(int64_t)s * (D + 2) + 2 + d] * w;
    }
  const int i = p / a.g, h = kv * a.g + p % a.g;
  out[((int64_t)i * a.hq + h) * D + d] = L > 0.f ? O / L : 0.f;
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
  if (a.q_bf16) {
    static const int per_cu = resident_per_cu(prefill_score_seg_kernel<D, R>, 256);
    const int nchunk = (a.P + 255) / 256;
    const int64_t cap = (int64_t)per_cu * device_cus() / ((int64_t)a.hkv * nchunk);
    hipLaunchKernelGGL((prefill_score_seg_kernel<D, R>),
                       dim3(grid_for(a.nl[1], SG_NODES, cap < 1 ? 1 : cap), (unsigned)(a.hkv * nchunk),
                            (unsigned)a.levels),
                       dim3(256), 0, st, a);
  } else {
    static const int per_cu = resident_per_cu(prefill_score_kernel<D, R>, 256);
    const int64_t cap = (int64_t)per_cu * device_cus() / a.hkv;
    hipLaunchKernelGGL((prefill_score_kernel<D, R>),
                       dim3(grid_for(a.nl[1], 4 * (16 / R), cap), (unsigned)a.hkv, (unsigned)a.levels), dim3(256), 0,
                       st, a);
  }
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

int prefill_attend_splits(int hkv, int P) {
  const int nchunk = (P + PA_CHUNK - 1) / PA_CHUNK;
  int s = PA_WGS / (hkv * nchunk);
  return s < 1 ? 1 : (s > PA_SPLITS ? PA_SPLITS : s);
}

hipError_t launch_prefill_attend(const PrefillArgs& a, float* part, float* out, int D, hipStream_t st) {
  const int nchunk = (a.P + PA_CHUNK - 1) / PA_CHUNK;
  const int ns = prefill_attend_splits(a.hkv, a.P);
  if (D == 64) {
    hipLaunchKernelGGL(prefill_attend_kernel<64>, dim3((unsigned)ns, (unsigned)(a.hkv * nchunk)), dim3(256), 0, st, a,
                       part, ns);
    hipLaunchKernelGGL(prefill_combine_kernel<64>, dim3((unsigned)a.P, (unsigned)a.hkv), dim3(64), 0, st, a,
                       (const float*)part, ns, out);
  } else if (D == 128) {
    hipLaunchKernelGGL(prefill_attend_kernel<128>, dim3((unsigned)ns, (unsigned)(a.hkv * nchunk)), dim3(256), 0, st,
                       a, part, ns);
    hipLaunchKernelGGL(prefill_combine_kernel<128>, dim3((unsigned)a.P, (unsigned)a.hkv), dim3(128), 0, st, a,
                       (const float*)part, ns, out);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace zha
