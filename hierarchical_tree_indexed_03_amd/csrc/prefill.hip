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
// is held in one of two ways for the passes that follow:
//   list  at most PS_LIST nodes: node ids and scores in LDS;
//   scan  a longer frontier: every pass reads the whole level from global memory (PS_UNROLL
//         loads in flight per thread), the frontier test from the parents' kept bitmap.
// Nodes outside the pair's tree score -inf and drop out.
constexpr int PS_UNROLL = 8;

__global__ __launch_bounds__(PS_THREADS, 4) void prefill_select_kernel(PrefillArgs a) {
  constexpr int NW = PS_THREADS / 64;
  __shared__ int32_t fl[PS_LIST];
  __shared__ float fs[PS_LIST];
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
    // past the list: the parents' kept bitmap goes to LDS (in the list's space) when it fits
    uint32_t* pbits = (uint32_t*)fl;
    const bool lds_bits = !list && !top && nwp <= PS_LIST;
    __syncthreads();
    if (lds_bits)
      for (int64_t w = tid; w < nwp; w += PS_THREADS) pbits[w] = ld_agent(kp + w);
    // kept marks: LDS bitmap (copied out at the end) or the global one; a listed frontier
    // sets bits one node at a time, so its bitmap starts cleared (the other modes write every
    // word in their classification pass)
    if (list) {
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
    // f(node, score) for every entry (score -inf outside the frontier)
    auto each = [&](auto&& f) {
      if (list) {
        for (int64_t k = tid; k < nf; k += PS_THREADS) f((int64_t)fl[k], fs[k]);
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

}  // namespace zha
