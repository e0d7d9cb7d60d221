// Router scoring.
//
// A node's score for a query is the max over its reference planes of q.s_j / sqrt(d) + c_j
// (news summary "Zyphra releases the ZHA sparse attention method", section "Building the
// tree"; blog "Zyphra Hierarchical Attention", section "Routing through the tree").
//
// GPU organisation.  The query heads of one GQA group share a KV head, hence a tree; the
// router keeps, per KV head and level, the UNION of the group's frontiers as a node list
// sorted by id with a bitmask of the heads whose frontier holds each node, so a node's
// planes are read once per group.  The score kernel writes every head's score of every
// union entry and the per-head max (ordered-integer atomics); the top levels, small enough
// to score whole, are scored in one launch over several levels.
#include "common.hpp"
#include "kernels.hpp"
#include "route_util.hpp"
#include "qk_tile.hpp"

// Score-kernel tuning: tiles in flight per wave (bf16 / FP4 planes).
#ifndef ZHA_SCORE_UN_BF16
#define ZHA_SCORE_UN_BF16 2
#endif

namespace zha {

// Dense scoring of the top levels: the level of this workgroup (grid z).  The largest level
// (the lowest) comes first, so its long-running workgroups are dispatched before the small
// levels' ones, which then fill the tail.
#ifndef ZHA_DENSE_LOW_FIRST
#define ZHA_DENSE_LOW_FIRST 1
#endif
__device__ __forceinline__ int dense_level(const RouteArgs& a) {
  return ZHA_DENSE_LOW_FIRST ? a.dense_lo + (int)blockIdx.z : a.level - (int)blockIdx.z;
}

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
  // list sizes: the top level's list, and every level selected top-down (a.dense_lo ..
  // L, all nodes scored); the others are written by the kernels that build their lists
  for (int64_t i = tid; i < (int64_t)(MAXL + 1) * a.hkv; i += nth) {
    const int lv = (int)(i / a.hkv);
    const int32_t n = (lv == L || (lv >= a.dense_lo && lv <= L && a.dense_lo >= 1)) ? (int32_t)a.nl[lv] : 0;
    a.dev.cnt[i] = n;
    a.dev.ucnt[i] = n;
  }
  if (a.dev.tick)
    for (int64_t i = tid; i < a.hkv; i += nth) a.dev.tick[i] = 0u;
}

// s_waitcnt vmcnt(n) with the export and LDS/scalar counters left free (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
// The scheduler may not move any instruction across it.
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | 0x0F70);
  __builtin_amdgcn_sched_barrier(0);
}

// ------------------------------------------------------------------ score
// Scores of the union frontier on fp32 MFMA: one 16x16 output tile = the 16 query-head rows
// (the group's heads, zero-padded) x 16 columns = 16/R nodes x R planes.  A node's score is
// the max over its R columns (plus the offsets c_j), taken across the R lanes of the node.
//
// Loading: each tile's 16 plane rows are read whole, RPI rows per load instruction (a row's
// 4D bytes by D/4 consecutive lanes, 16 bytes each), so every instruction reads whole
// 512-byte rows (d 128) instead of one 64-byte piece of each of 16 rows; the rows go through
// LDS (rows padded by 16 bytes, so the MFMA-layout reads hit distinct banks) into the MFMA
// operand layout: lane (column c, group kg) takes the pieces [64i + 16kg, +16) of row c, and
// Q uses the same permutation of the contraction.
//
// Pipeline per wave: the next tile's rows and offsets are loaded while the current tile is
// scored, and (list mode) the node ids of the tile after it.  Every load is unconditional at
// a clamped index (past the list's end: its last entry) and validity is applied where the
// values are used, so no load waits on another; a tile's scores are stored one pass later,
// after the next pass's loads, so each pass's single wait finds every operation it waits for
// as old as the pass.  DENSE: every node of the level (grid z: the level), no list.
template <int D, int R, bool DENSE>
__global__ __launch_bounds__(256) void route_score_kernel(RouteArgs a) {
  constexpr int NPT = 16 / R;                 // nodes per 16-column tile
  constexpr int NI = D / 16;                  // float4 MFMA operands per lane per tile
  constexpr int LPR = D / 4;                  // lanes per row in a load instruction
  constexpr int RPI = 64 / LPR;               // rows per load instruction
  constexpr int NLD = 16 / RPI;               // load instructions per tile
  constexpr int RS = D + 4;                   // LDS row stride in floats
  __shared__ __align__(16) float stg[4][16 * RS];
  __shared__ float red[4][16];
  // the wave index through readfirstlane, so the compiler sees the tile loop as uniform
  const int kv = blockIdx.y, lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, kg = lane >> 4;
  const int slot = col / R, plane = col % R;
  const int lrow = lane / LPR, lcol = (lane % LPR) * 4;
  const int lv = DENSE ? dense_level(a) : a.level;
  const int64_t cnt = DENSE ? a.nl[lv] : a.dev.cnt[lv * a.hkv + kv];
  const int64_t cap = a.dev.ncap[lv];
  const int64_t nl = a.nl[lv];
  const int32_t* nodes = a.dev.node[lv] + kv * cap;
  const uint32_t* masks = a.dev.mask[lv] + kv * cap;
  const float* S = a.dev.s[lv] + (int64_t)kv * cap * R * D;
  const float* C = a.dev.c[lv] + (int64_t)kv * cap * R;
  float* out = a.dev.score[lv] + (int64_t)kv * GMAX * cap;
  float* W = stg[wave];
  const int g = a.g;
  ZHA_CHECK(a.dev, cnt <= cap, CHK_LIST_SIZE);

  float qa[NI][4];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
    if (col < g) x = *(const float4*)(a.dev.qf + (int64_t)(kv * g + col) * D + 16 * i + 4 * kg);
    qa[i][0] = x.x; qa[i][1] = x.y; qa[i][2] = x.z; qa[i][3] = x.w;
  }
  float runmax[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};

  const int64_t ntiles = (cnt + NPT - 1) / NPT;
  const int64_t tstride = (int64_t)gridDim.x * 4;
  const int64_t tfirst = (int64_t)blockIdx.x * 4 + wave;
  auto clamp_e = [&](int64_t e) __attribute__((always_inline)) { return e < cnt ? e : cnt - 1; };
  auto clamp_n = [&](int64_t n) __attribute__((always_inline)) { return n < 0 ? (int64_t)0 : (n < nl ? n : nl - 1); };

  // list mode: the node of each of the lane's NLD load rows, and its MFMA slot's node and
  // head mask (row r of tile t: entry t * NPT + r / R)
  int32_t lid[NLD], sid;
  uint32_t smk;
  auto load_ids = [&](int64_t t) __attribute__((always_inline)) {
    if constexpr (!DENSE) {
#pragma unroll
      for (int i = 0; i < NLD; ++i) lid[i] = nodes[clamp_e(t * NPT + (lrow + RPI * i) / R)];
      const int64_t es = clamp_e(t * NPT + slot);
      sid = nodes[es];
      smk = masks[es];
    }
  };
  // a tile's rows and the lane's offset c (rows of entries past the list read its last one)
  u32x4 ld[NLD];
  float rcj;
  uint32_t rmk;
  auto fetch = [&](int64_t t) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int r = lrow + RPI * i;
      const int64_t nd = DENSE ? clamp_e(t * NPT + r / R) : clamp_n(lid[i]);
      ZHA_CHECK(a.dev, DENSE || t * NPT + r / R >= cnt || (lid[i] >= 0 && lid[i] < nl), CHK_NODE_RANGE);
      ld[i] = *(const u32x4*)(S + (nd * R + r % R) * D + lcol);
    }
    const int64_t es = t * NPT + slot;
    const int64_t nd = DENSE ? clamp_e(es) : clamp_n(sid);
    rcj = C[nd * R + plane];
    // dense: every head's score of an entry of the level; list: the heads holding the entry
    rmk = es < cnt ? (DENSE ? 0xffffffffu : smk) : 0u;
  };
  // scores stored one pass late (lane (col, kg) with plane 0: heads 4kg..4kg+3 of its slot)
  float pv[4] = {0.f, 0.f, 0.f, 0.f};
  uint32_t pmk = 0u;
  int64_t pent = 0;
  auto store_pending = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int h = kg * 4 + e;
      if (plane == 0 && h < g && ((pmk >> h) & 1u)) out[(int64_t)h * cap + pent] = pv[e];
    }
  };

  if (tfirst < ntiles) {
    load_ids(tfirst);
    fetch(tfirst);
    load_ids(tfirst + tstride);
    for (int64_t t = tfirst; t < ntiles; t += tstride) {
      wait_vm<0>();
#pragma unroll
      for (int i = 0; i < NLD; ++i) *(u32x4*)(W + (lrow + RPI * i) * RS + lcol) = ld[i];
      const float cj = rcj;
      const uint32_t mk = rmk;
      wave_sync_lds();
      fetch(t + tstride);
      load_ids(t + 2 * tstride);
      store_pending();
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const float4 sb = *(const float4*)(W + col * RS + 16 * i + 4 * kg);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[i][0], sb.x, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[i][1], sb.y, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[i][2], sb.z, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[i][3], sb.w, acc, 0, 0, 0);
      }
      wave_sync_lds();
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = acc[e] + cj;
#pragma unroll
      for (int off = 1; off < R; off <<= 1)
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = fmaxf(v[e], __shfl_xor(v[e], off));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pv[e] = v[e];
        // the per-head max of list mode (dense levels take theirs in the selection)
        if (!DENSE && ((mk >> (kg * 4 + e)) & 1u)) runmax[e] = fmaxf(runmax[e], v[e]);
      }
      pmk = mk;
      pent = t * NPT + slot;
    }
    store_pending();
  }
  if constexpr (!DENSE) {
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
}


// ------------------------------------------------------------------ bf16 router planes
// A 16-row tile of bf16 plane rows (row c = node slot c / R, plane c % R) for one lane:
// the contiguous D/4 slice [kg D/4, (kg+1) D/4) of its row, in the operand layout of
// Qk<TQ, D> (bf16 as loaded; fp32 queries take the values widened to fp32).
template <typename TQ, int D> struct PlaneRow;
template <int D> struct PlaneRow<bf16_t, D> {
  static constexpr int NL = Qk<bf16_t, D>::NL;
  __device__ static void load(const bf16_t* row, int kg, bool ok, uint4* k) {
#pragma unroll
    for (int i = 0; i < NL; ++i) k[i] = ok ? *(const uint4*)(row + kg * (D / 4) + i * 8) : make_uint4(0, 0, 0, 0);
  }
};
template <int D> struct PlaneRow<float, D> {
  static constexpr int NL = Qk<float, D>::NL;
  __device__ static void load(const bf16_t* row, int kg, bool ok, uint4* k) {
#pragma unroll
    for (int i = 0; i < NL / 2; ++i) {
      const uint4 w = ok ? *(const uint4*)(row + kg * (D / 4) + i * 8) : make_uint4(0, 0, 0, 0);
      k[2 * i] = make_uint4(w.x << 16, w.x & 0xffff0000u, w.y << 16, w.y & 0xffff0000u);
      k[2 * i + 1] = make_uint4(w.z << 16, w.z & 0xffff0000u, w.w << 16, w.w & 0xffff0000u);
    }
  }
};

// The same slice of an MX FP4 row: D/8 bytes of E2M1 codes (element 2i in the low nibble of
// byte i) and the scale byte of the slice's 32-element block, widened on the fly to bf16 by
// the scaled conversion (code value times 2^(scale - 127), exact in bf16).
__device__ __forceinline__ uint4 fp4x8_to_bf16(uint32_t w, float sc) {
  return make_uint4(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3)));
}
template <int D>
__device__ __forceinline__ void load_fp4_slice(const uint8_t* row, const uint8_t* xrow, int kg, bool ok,
                                               uint4 (&b)[D / 32]) {
  uint32_t w[D / 32];
  if constexpr (D == 128) {
    const uint4 t = ok ? *(const uint4*)(row + kg * 16) : make_uint4(0, 0, 0, 0);
    w[0] = t.x; w[1] = t.y; w[2] = t.z; w[3] = t.w;
  } else {
    const uint2 t = ok ? *(const uint2*)(row + kg * 8) : make_uint2(0, 0);
    w[0] = t.x; w[1] = t.y;
  }
  const uint32_t sb = ok ? (uint32_t)xrow[(kg * (D / 4)) / 32] : 0u;
  const float sc = __uint_as_float(sb << 23);          // 2^(sb - 127); an all-zero block: 0
#pragma unroll
  for (int i = 0; i < D / 32; ++i) b[i] = fp4x8_to_bf16(w[i], sc);
}
template <typename TQ, int D> struct Fp4Row;
template <int D> struct Fp4Row<bf16_t, D> {
  static constexpr int NL = Qk<bf16_t, D>::NL;
  __device__ static void load(const uint8_t* row, const uint8_t* xrow, int kg, bool ok, uint4* k) {
    uint4 b[D / 32];
    load_fp4_slice<D>(row, xrow, kg, ok, b);
#pragma unroll
    for (int i = 0; i < NL; ++i) k[i] = b[i];
  }
};
template <int D> struct Fp4Row<float, D> {
  static constexpr int NL = Qk<float, D>::NL;
  __device__ static void load(const uint8_t* row, const uint8_t* xrow, int kg, bool ok, uint4* k) {
    uint4 b[D / 32];
    load_fp4_slice<D>(row, xrow, kg, ok, b);
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
      k[2 * i] = make_uint4(b[i].x << 16, b[i].x & 0xffff0000u, b[i].y << 16, b[i].y & 0xffff0000u);
      k[2 * i + 1] = make_uint4(b[i].z << 16, b[i].z & 0xffff0000u, b[i].w << 16, b[i].w & 0xffff0000u);
    }
  }
};

// Scores from the bf16 copies of s: the tile Q (16 heads x D) . P^T (D x 16 plane rows) on
// MFMA with the raw query as the A operand (bf16 x bf16 products are exact in the fp32
// accumulator; fp32 queries take the fp32 MFMA on planes widened to fp32), then
// sigma * acc + c_j.  Plane row c = (node slot c / R, plane c % R).  A lane (column col,
// group kg) loads row col and receives that row's scores for heads 4kg..4kg+3, so a node's
// id, offset and head mask are read by the lanes that read its planes; the max over a
// node's R planes runs across R neighbouring lanes.  The next pass's node ids and masks are
// loaded before this pass's planes.
// With FP4 = true the rows are the MX FP4 copies, widened to bf16 as they are loaded.
template <typename TQ, int D, int R, bool FP4>
__global__ __launch_bounds__(256) void route_score_bf16_kernel(RouteArgs a) {
  constexpr int NPT = 16 / R;                 // nodes per 16-row tile
  constexpr int UN = ZHA_SCORE_UN_BF16;       // tiles in flight per wave
  constexpr int NL = PlaneRow<TQ, D>::NL;
  __shared__ float red[4][16];
  const int kv = blockIdx.y, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, kg = lane >> 4;
  const int slot = col / R, plane = col % R;
  const bool dense = a.dense != 0;            // every node of the level, no list
  const int lv = dense ? dense_level(a) : a.level;
  const int64_t cnt = dense ? a.nl[lv] : a.dev.cnt[lv * a.hkv + kv];
  const int64_t cap = a.dev.ncap[lv];
  const int32_t* nodes = a.dev.node[lv] + kv * cap;
  const uint32_t* masks = a.dev.mask[lv] + kv * cap;
  const bf16_t* S = FP4 ? nullptr : a.dev.sq[lv] + (int64_t)kv * cap * R * D;
  const uint8_t* S4 = FP4 ? a.dev.s4[lv] + (int64_t)kv * cap * R * (D / 2) : nullptr;
  const uint8_t* X4 = FP4 ? a.dev.s4x[lv] + (int64_t)kv * cap * R * (D / 32) : nullptr;
  const float* C = a.dev.c[lv] + (int64_t)kv * cap * R;
  float* out = a.dev.score[lv] + (int64_t)kv * GMAX * cap;
  const int g = a.g;
  const float sigma = a.sigma;

  // the A operand: head col's query, slice kg of the permuted contraction (zero past g)
  Qk<TQ, D> qk;
  qk.load_q((const TQ*)a.q + (int64_t)kv * g * D, g, col, kg);
  float runmax[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};   // heads 4kg..4kg+3

  const int64_t ntiles = (cnt + NPT - 1) / NPT;
  const int64_t tstride = (int64_t)gridDim.x * 4 * UN;
  int32_t nid[UN];                            // the lane's node per tile of the pass; -1 none
  uint32_t nmk[UN];
  auto load_ids = [&](int64_t t0, int32_t (&nd)[UN], uint32_t (&mk)[UN]) {
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int64_t e = (t0 + u) * NPT + slot;
      const bool ok = (t0 + u) < ntiles && e < cnt;
      mk[u] = (ok && !dense) ? masks[e] : 0u;   // dense: the max is taken later
      // list mode: an entry of no head's frontier (mask 0) is not read
      nd[u] = (ok && (dense || mk[u] != 0u)) ? (dense ? (int32_t)e : nodes[e]) : -1;
    }
  };
  const int64_t tfirst = ((int64_t)blockIdx.x * 4 + wave) * UN;
  if (tfirst < ntiles) load_ids(tfirst, nid, nmk);
  for (int64_t t0 = tfirst; t0 < ntiles; t0 += tstride) {
    int32_t ncur[UN];
    uint32_t mcur[UN];
#pragma unroll
    for (int u = 0; u < UN; ++u) { ncur[u] = nid[u]; mcur[u] = nmk[u]; }
    if (t0 + tstride < ntiles) load_ids(t0 + tstride, nid, nmk);
    uint4 kf[UN][NL];
    float cj[UN];
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const bool ok = ncur[u] >= 0;
      const int64_t nd = ok ? ncur[u] : 0;
      if constexpr (FP4)
        Fp4Row<TQ, D>::load(S4 + (nd * R + plane) * (D / 2), X4 + (nd * R + plane) * (D / 32), kg, ok, kf[u]);
      else
        PlaneRow<TQ, D>::load(S + (nd * R + plane) * D, kg, ok, kf[u]);
      cj[u] = ok ? C[nd * R + plane] : -INFINITY;
    }
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      if constexpr (sizeof(TQ) == 2) {
#pragma unroll
        for (int i = 0; i < NL; ++i)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qk.q[i], __builtin_bit_cast(bf16x8, kf[u][i]), acc, 0, 0, 0);
      } else {
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qk.q[4 * i + 0], __uint_as_float(kf[u][i].x), acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qk.q[4 * i + 1], __uint_as_float(kf[u][i].y), acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qk.q[4 * i + 2], __uint_as_float(kf[u][i].z), acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qk.q[4 * i + 3], __uint_as_float(kf[u][i].w), acc, 0, 0, 0);
        }
      }
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = sigma * acc[e] + cj[u];
#pragma unroll
      for (int off = 1; off < R; off <<= 1)
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = fmaxf(v[e], __shfl_xor(v[e], off));
      const int64_t ent = (t0 + u) * NPT + slot;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int h = kg * 4 + e;
        if (ncur[u] >= 0 && plane == 0 && h < g && (dense || ((mcur[u] >> h) & 1u))) out[(int64_t)h * cap + ent] = v[e];
        if ((mcur[u] >> h) & 1u) runmax[e] = fmaxf(runmax[e], v[e]);
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


// The same scores with the tile transposed, S = P (16 plane rows x D) . Q^T (D x 16 heads):
// lane (head col, group kg) holds rows 4kg..4kg+3 for head col, so with R >= 4 a node's
// planes come four to a lane and the max over planes is three in-lane steps and R/8
// cross-lane ones (R 16: 2 shuffles per head value instead of 4).  Used for R >= 8.
template <typename TQ, int D, int R>
__global__ __launch_bounds__(256) void route_score_bf16_rows_kernel(RouteArgs a) {
  constexpr int NPT = 16 / R;                 // nodes per 16-row tile
  constexpr int UN = ZHA_SCORE_UN_BF16;       // tiles in flight per wave
  constexpr int NL = Qk<TQ, D>::NL;
  constexpr int RL = R < 4 ? R : 4;           // rows of one node within a lane's 4 rows
  constexpr int NPL = 4 / RL;                 // nodes within a lane's 4 rows
  __shared__ float red[4][16];
  const int kv = blockIdx.y, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, kg = lane >> 4;
  const bool dense = a.dense != 0;            // every node of the level, no list
  const int lv = dense ? dense_level(a) : a.level;
  const int64_t cnt = dense ? a.nl[lv] : a.dev.cnt[lv * a.hkv + kv];
  const int64_t cap = a.dev.ncap[lv];
  const int32_t* nodes = a.dev.node[lv] + kv * cap;
  const uint32_t* masks = a.dev.mask[lv] + kv * cap;
  const bf16_t* S = a.dev.sq[lv] + (int64_t)kv * cap * R * D;
  const float* C = a.dev.c[lv] + (int64_t)kv * cap * R;
  float* out = a.dev.score[lv] + (int64_t)kv * GMAX * cap;
  const int g = a.g;
  const float sigma = a.sigma;

  Qk<TQ, D> qk;
  qk.load_q((const TQ*)a.q + (int64_t)kv * g * D, g, col, kg);
  float runmax = -INFINITY;                   // head col

  const int64_t ntiles = (cnt + NPT - 1) / NPT;
  for (int64_t t0 = ((int64_t)blockIdx.x * 4 + wave) * UN; t0 < ntiles; t0 += (int64_t)gridDim.x * 4 * UN) {
    uint4 kf[UN][NL];
    float cj[UN][4];
    int64_t eo[UN][NPL];                      // union entries of the lane's output nodes
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const bool tok = (t0 + u) < ntiles;
      // the lane's load row `col`
      const int64_t e_row = (t0 + u) * NPT + col / R;
      // list mode: an entry of no head's frontier (mask 0) is not read
      const bool okr = tok && e_row < cnt && (dense || masks[e_row] != 0u);
      const int64_t nrow = okr ? (dense ? e_row : (int64_t)nodes[e_row]) : 0;
      PlaneRow<TQ, D>::load(S + (nrow * R + col % R) * D, kg, okr, kf[u]);
      // the lane's output rows 4kg + e
#pragma unroll
      for (int n = 0; n < NPL; ++n) {
        const int r = 4 * kg + n * RL;
        const int64_t e = (t0 + u) * NPT + r / R;
        const bool ok = tok && e < cnt;
        eo[u][n] = ok ? e : -1;
        const int64_t nd = ok ? (dense ? e : (int64_t)nodes[e]) : 0;
        if constexpr (RL == 4) {
          const float4 c4 = ok ? *(const float4*)(C + nd * R + r % R) : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
          cj[u][0] = c4.x; cj[u][1] = c4.y; cj[u][2] = c4.z; cj[u][3] = c4.w;
        } else {
#pragma unroll
          for (int i = 0; i < RL; ++i) cj[u][n * RL + i] = ok ? C[nd * R + i] : -INFINITY;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const f32x4 acc = qk.mma(kf[u]);        // acc[e]: row 4kg+e, head col
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = sigma * acc[e] + cj[u][e];
#pragma unroll
      for (int o = 1; o < RL; o <<= 1)
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = fmaxf(v[e], v[e ^ o]);
#pragma unroll
      for (int o = 16; o < 4 * R; o <<= 1)
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = fmaxf(v[e], __shfl_xor(v[e], o));
#pragma unroll
      for (int n = 0; n < NPL; ++n) {
        const int64_t e = eo[u][n];
        const bool writer = ((4 * kg) % R) == 0;    // the node's first lane group
        const uint32_t mk = (e >= 0 && !dense) ? masks[e] : 0u;   // dense: max taken later
        if (e >= 0 && writer && col < g && (dense || ((mk >> col) & 1u))) out[(int64_t)col * cap + e] = v[n * RL];
        if ((mk >> col) & 1u) runmax = fmaxf(runmax, v[n * RL]);
      }
    }
  }
  // per-head max over the wave's lane groups, then over the waves
  runmax = fmaxf(runmax, __shfl_xor(runmax, 16));
  runmax = fmaxf(runmax, __shfl_xor(runmax, 32));
  if (kg == 0) red[wave][col] = runmax;
  __syncthreads();
  if (threadIdx.x < g) {
    const int gi = threadIdx.x;
    const float m = fmaxf(fmaxf(red[0][gi], red[1][gi]), fmaxf(red[2][gi], red[3][gi]));
    if (m > -INFINITY) atomicMax(&a.dev.qs[lv * a.hq + kv * g + gi].maxkey, f2key(m));
  }
}


// ------------------------------------------------------------------ key-form level 1
// A level-1 plane's s_j is the softmax-weighted mean of its block's keys (weights w_jt over
// the block's tokens at r_j), so q.s_j / sqrt(d) = sum_t w_jt (q.k_t / sqrt(d)): the scores
// of a block follow from the group's logits on its b keys and the R x b stored weights.
// Per 16-token tile (16/b nodes): the logits tile S^T = K.Q^T (bf16 MFMA, tokens x heads),
// transposed through LDS, then per node one fp32 MFMA per 4 tokens, [planes x tokens] x
// [tokens x heads] accumulated onto c_j, so each lane holds 4 planes of one head.  The max
// over a node's planes is 3 in-lane maxima and a maximum over the 4 lane rows; the tile's
// nodes share the cross-row steps (a butterfly on the gfx950 row swaps), which leave each
// row with the full maxima of its own nodes.

template <int D, int R, int B>
__global__ __launch_bounds__(256, B >= 4 ? 4 : 1) void route_score_keys_kernel(RouteArgs a) {
  constexpr int NPT = 16 / B;                 // nodes per 16-token tile
  constexpr int KS = (B + 3) / 4;             // fp32 MFMA steps per node
  constexpr int NK = Qk<bf16_t, D>::NL;
  constexpr int NC = NPT >= 4 ? NPT / 4 : 1;  // node maxima per lane after the row steps
  constexpr int NROW = NPT >= 4 ? 4 : NPT;    // lane rows that hold distinct nodes
  __shared__ float Lt[4][16][17];             // per wave: logits [head][token]
  __shared__ float red[4][16];
  // the wave index through readfirstlane, so the compiler sees the tile loop as uniform
  const int kv = blockIdx.y, lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, kg = lane >> 4;
  const int lv = 1;
  const int cnt = (int)a.dev.cnt[lv * a.hkv + kv];
  const int64_t cap = a.dev.ncap[lv];
  const int nl = (int)a.nl[lv];
  const int32_t* nodes = a.dev.node[lv] + kv * cap;
  const uint32_t* masks = a.dev.mask[lv] + kv * cap;
  const bf16_t* Kc = (const bf16_t*)a.K + (int64_t)kv * a.kcap * D;
  const float* W = a.dev.w1 + (int64_t)kv * cap * R * B;
  const float* C = a.dev.c[lv] + (int64_t)kv * cap * R;
  float* out = a.dev.score[lv] + (int64_t)kv * GMAX * cap;
  const int g = a.g;
  const int N = (int)a.N;

  Qk<bf16_t, D> qk;
  qk.load_q((const bf16_t*)a.q + (int64_t)kv * g * D, g, col, kg);
  float runmax = -INFINITY;                   // head `col`, over this lane row's nodes

  const int ntiles = (cnt + NPT - 1) / NPT;
  const int tstride = (int)gridDim.x * 4;
  const int tfirst = (int)blockIdx.x * 4 + wave;

  // Two-stage pipeline per wave: the node ids of the tile after next and the keys, weights
  // and c of the next tile are in flight while the current tile is scored.  Every load is
  // unconditional at a clamped index (past the list's end: its last entry, a cache hit);
  // validity is applied where the values are used, so no load waits on another.  The ids
  // are per-lane vector loads (lane `col` holds the entry of its token row); a node's id and
  // head mask reach the wave as the value of lane n * B, so no scalar-cache load (whose wait
  // would share the LDS counter) sits in the pass.
  int32_t rid;
  uint32_t rmk;
  auto load_ids = [&](int t) {
    const int er = min(t * NPT + col / B, cnt - 1);
    rid = nodes[er];
    rmk = masks[er];
  };
  // a tile's operands and the head masks of its nodes
  struct Tile {
    uint4 kf[NK];
    float wv[NPT][KS];
    f32x4 cj[NPT];
    uint32_t mk[NPT];                         // 0 past the list's end
  };
  // Token rows past the cache's end (a partial last block) read the last key: their weights
  // are stored as exact zeros, so they add nothing to any plane's score.  Rows of entries
  // that no head holds feed only scores that are never stored.
  auto load_tile = [&](int t, Tile& x) {
    // the tile's 16 token rows: token `col` of node col / B
    const int tok = min(max(rid, 0), nl - 1) * B + col % B;
    Qk<bf16_t, D>::load_k(Kc + (int64_t)min(tok, N - 1) * D, kg, x.kf);
#pragma unroll
    for (int n = 0; n < NPT; ++n) {
      const int32_t nid = __builtin_amdgcn_readlane(rid, n * B);
      x.mk[n] = t * NPT + n < cnt ? (uint32_t)__builtin_amdgcn_readlane((int32_t)rmk, n * B) : 0u;
      ZHA_CHECK(a.dev, x.mk[n] == 0u || (nid >= 0 && nid < nl), CHK_NODE_RANGE);
      const int64_t nd = min(max(nid, 0), nl - 1);
      // A operand: lane (plane col, token 4s + kg) holds w[plane][token]
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int k = 4 * s + kg;
        x.wv[n][s] = W[(nd * R + min(col, R - 1)) * B + min(k, B - 1)];
      }
      // accumulator: c of planes 4kg..4kg+3 (absent planes -inf where used)
      if constexpr (R >= 4) {
        const float4 c4 = *(const float4*)(C + nd * R + min(4 * kg, R - 4));
        x.cj[n][0] = c4.x; x.cj[n][1] = c4.y; x.cj[n][2] = c4.z; x.cj[n][3] = c4.w;
      } else {
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) x.cj[n][e4] = C[nd * R + min(4 * kg + e4, R - 1)];
      }
    }
  };
  // A tile's scores are stored one pass later, after the next pass's loads are issued: the
  // wait at a pass's start then finds those stores as old as the loads it waits for, instead
  // of waiting for stores issued just before it.  Lane (col, row kg) stores head col's score
  // of the nodes its row holds.
  float pv[NC];
  uint32_t pmk[NC];
  int pt = 0;
#pragma unroll
  for (int i = 0; i < NC; ++i) { pv[i] = 0.f; pmk[i] = 0u; }
  auto store_pending = [&]() {
#pragma unroll
    for (int i = 0; i < NC; ++i)
      if (((pmk[i] >> col) & 1u) && kg < NROW && col < g)
        out[(int64_t)col * cap + pt * NPT + key_row_node<NPT>(i, kg)] = pv[i];
  };
  auto score_tile = [&](int t, const Tile& x) {
    const f32x4 st = qk.mma(x.kf);              // S^T[token 4kg+e][head col]
#pragma unroll
    for (int e = 0; e < 4; ++e) Lt[wave][col][kg * 4 + e] = a.sigma * st[e];
    wave_sync_lds();
    float m[NPT];
#pragma unroll
    for (int n = 0; n < NPT; ++n) {
      f32x4 acc;
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) acc[e4] = 4 * kg + e4 < R ? x.cj[n][e4] : -INFINITY;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int k = 4 * s + kg;
        // B operand: lane (head col, token k) holds the logit
        const float lg = k < B ? Lt[wave][col][n * B + k] : 0.f;
        const float w = col < R && k < B ? x.wv[n][s] : 0.f;
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(w, lg, acc, 0, 0, 0);
      }
      // acc[e] = score of plane 4kg+e for head col
      m[n] = fmaxf(fmaxf(acc[0], acc[1]), fmaxf(acc[2], acc[3]));
    }
    float v[NC];
    key_row_max<NPT>(m, v);
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      // the head mask of this row's node: NPT wave-uniform values, picked by the row
      uint32_t mk = 0u;
#pragma unroll
      for (int n = 0; n < NPT; ++n) mk = key_row_node<NPT>(i, kg) == n ? x.mk[n] : mk;
      pv[i] = v[i];
      pmk[i] = mk;
      if (((mk >> col) & 1u) && kg < NROW) runmax = fmaxf(runmax, v[i]);
    }
    pt = t;
    wave_sync_lds();
  };

  // Each pass starts with an explicit wait for all of the previous pass's memory operations
  // (its loads and the stores issued beside them, all as old as the pass); the compiler's
  // own counting across the two alternating halves would otherwise wait inside the pass
  // for some of the loads just issued.
  if (tfirst < ntiles) {
    Tile ta, tb;
    load_ids(tfirst);
    load_tile(tfirst, ta);
    load_ids(tfirst + tstride);
    for (int t = tfirst; t < ntiles; t += 2 * tstride) {
      wait_vm<0>();
      load_tile(t + tstride, tb);
      load_ids(t + 2 * tstride);
      store_pending();
      score_tile(t, ta);
      if (t + tstride >= ntiles) break;
      wait_vm<0>();
      load_tile(t + 2 * tstride, ta);
      load_ids(t + 3 * tstride);
      store_pending();
      score_tile(t + tstride, tb);
    }
    store_pending();
  }
  runmax = fmaxf(runmax, __shfl_xor(runmax, 16));
  runmax = fmaxf(runmax, __shfl_xor(runmax, 32));
  if (kg == 0) red[wave][col] = runmax;
  __syncthreads();
  if (threadIdx.x < g) {
    const int gi = threadIdx.x;
    const float m = fmaxf(fmaxf(red[0][gi], red[1][gi]), fmaxf(red[2][gi], red[3][gi]));
    if (m > -INFINITY) atomicMax(&a.dev.qs[lv * a.hq + kv * g + gi].maxkey, f2key(m));
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

// Score grids hold one wave of resident workgroups over the KV heads (the node loop is
// strided), so no workgroup of a second, partial wave trails the launch.
template <typename TQ, int D, int R>
static void launch_score_bf16(const RouteArgs& a, int nlev, int64_t nodes, hipStream_t st) {
  constexpr int NPB = 4 * (16 / R) * ZHA_SCORE_UN_BF16;   // nodes per block pass
  if constexpr (R >= 8) {
    static const int per_cu = resident_per_cu(route_score_bf16_rows_kernel<TQ, D, R>, 256);
    const int64_t cap = (int64_t)per_cu * device_cus() / a.hkv;
    hipLaunchKernelGGL((route_score_bf16_rows_kernel<TQ, D, R>), dim3(grid_for(nodes, NPB, cap), (unsigned)a.hkv, (unsigned)nlev),
                       dim3(256), 0, st, a);
  } else {
    static const int per_cu = resident_per_cu(route_score_bf16_kernel<TQ, D, R, false>, 256);
    const int64_t cap = (int64_t)per_cu * device_cus() / a.hkv;
    hipLaunchKernelGGL((route_score_bf16_kernel<TQ, D, R, false>), dim3(grid_for(nodes, NPB, cap), (unsigned)a.hkv, (unsigned)nlev),
                       dim3(256), 0, st, a);
  }
}

template <typename TQ, int D, int R>
static void launch_score_fp4(const RouteArgs& a, int nlev, int64_t nodes, hipStream_t st) {
  constexpr int NPB = 4 * (16 / R) * ZHA_SCORE_UN_BF16;   // nodes per block pass
  static const int per_cu = resident_per_cu(route_score_bf16_kernel<TQ, D, R, true>, 256);
  const int64_t cap = (int64_t)per_cu * device_cus() / a.hkv;
  hipLaunchKernelGGL((route_score_bf16_kernel<TQ, D, R, true>), dim3(grid_for(nodes, NPB, cap), (unsigned)a.hkv, (unsigned)nlev),
                     dim3(256), 0, st, a);
}

template <int D, int R>
static void launch_score_planes(const RouteArgs& a, int nlev, int64_t nodes, hipStream_t st) {
  if (a.planes == 2) {
    if (a.q_bf16) launch_score_fp4<bf16_t, D, R>(a, nlev, nodes, st);
    else launch_score_fp4<float, D, R>(a, nlev, nodes, st);
    return;
  }
  if (a.planes == 1) {
    if (a.q_bf16) launch_score_bf16<bf16_t, D, R>(a, nlev, nodes, st);
    else launch_score_bf16<float, D, R>(a, nlev, nodes, st);
    return;
  }
  constexpr int NPB = 4 * (16 / R);   // nodes per block pass
  if (a.dense) {
    static const int per_cu = resident_per_cu(route_score_kernel<D, R, true>, 256);
    const int64_t cap = (int64_t)per_cu * device_cus() / a.hkv;
    hipLaunchKernelGGL((route_score_kernel<D, R, true>), dim3(grid_for(nodes, NPB, cap), (unsigned)a.hkv, (unsigned)nlev),
                       dim3(256), 0, st, a);
  } else {
    static const int per_cu = resident_per_cu(route_score_kernel<D, R, false>, 256);
    const int64_t cap = (int64_t)per_cu * device_cus() / a.hkv;
    hipLaunchKernelGGL((route_score_kernel<D, R, false>), dim3(grid_for(nodes, NPB, cap), (unsigned)a.hkv, (unsigned)nlev),
                       dim3(256), 0, st, a);
  }
}

template <int D, int R, int B>
static void launch_score_keys(const RouteArgs& a, hipStream_t st) {
  constexpr int NPB = 4 * (16 / B);   // nodes per block pass
  static const int per_cu = resident_per_cu(route_score_keys_kernel<D, R, B>, 256);
  const int64_t cap = (int64_t)per_cu * device_cus() / a.hkv;
  hipLaunchKernelGGL((route_score_keys_kernel<D, R, B>), dim3(grid_for(a.nlevel, NPB, cap), (unsigned)a.hkv), dim3(256),
                     0, st, a);
}

hipError_t launch_route_score(const RouteArgs& a, int D, int R, hipStream_t st) {
  if (a.key_form && a.level == 1 && !a.dense) {
#define ZHA_KCASE(DD, RR, BB) else if (D == DD && R == RR && a.b == BB) launch_score_keys<DD, RR, BB>(a, st);
#define ZHA_KCASES(DD, RR) ZHA_KCASE(DD, RR, 2) ZHA_KCASE(DD, RR, 4) ZHA_KCASE(DD, RR, 8) ZHA_KCASE(DD, RR, 16)
    if (false) {}
    ZHA_KCASES(64, 2) ZHA_KCASES(64, 4) ZHA_KCASES(64, 8) ZHA_KCASES(64, 16)
    ZHA_KCASES(128, 2) ZHA_KCASES(128, 4) ZHA_KCASES(128, 8) ZHA_KCASES(128, 16)
    else return hipErrorInvalidValue;
#undef ZHA_KCASES
#undef ZHA_KCASE
    return hipGetLastError();
  }
#define ZHA_CASE(DD, RR) else if (D == DD && R == RR) launch_score_planes<DD, RR>(a, 1, a.nlevel, st);
  if (false) {}
  ZHA_CASE(64, 1) ZHA_CASE(64, 2) ZHA_CASE(64, 4) ZHA_CASE(64, 8) ZHA_CASE(64, 16)
  ZHA_CASE(128, 1) ZHA_CASE(128, 2) ZHA_CASE(128, 4) ZHA_CASE(128, 8) ZHA_CASE(128, 16)
  else return hipErrorInvalidValue;
#undef ZHA_CASE
  return hipGetLastError();
}

template <int D, int R>
static void launch_dense_score_t(const RouteArgs& a, int nlev, hipStream_t st) {
  int64_t mx = 0;
  for (int l = a.dense_lo; l <= a.level; ++l) mx = a.nl[l] > mx ? a.nl[l] : mx;
  launch_score_planes<D, R>(a, nlev, mx, st);
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

}  // namespace zha
