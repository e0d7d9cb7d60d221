// Frontier expansion: the kept nodes' children become the next level's union list (in id
// order), or the kept level-1 blocks become the gather list.  Blog "Zyphra Hierarchical
// Attention", section "Routing through the tree" (only kept nodes are expanded).
// Two launches: per-chunk output counts, then compaction and emission at the chunk's
// offset.  List sizes stay on the device.
#include "common.hpp"
#include "kernels.hpp"
#include "route_util.hpp"

namespace zha {

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
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    a.dev.cnt[out_lv * a.hkv + kv] = red2[0] + red2[1] + red2[2] + red2[3];
    a.dev.ucnt[out_lv * a.hkv + kv] = red2[0] + red2[1] + red2[2] + red2[3];
  }
  const int32_t total = total_s;
  const int64_t ocap = a.dev.ncap[out_lv];
  ZHA_CHECK(a.dev, (int64_t)base + total <= ocap, CHK_EXPAND_RANGE);
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

// ------------------------------------------------------------------ launchers
hipError_t launch_route_expand(const RouteArgs& a, hipStream_t st) {
  const unsigned nch = (unsigned)((a.nlevel + EXPAND_CHUNK - 1) / EXPAND_CHUNK);
  dim3 grid(nch < 1 ? 1 : nch, (unsigned)a.hkv);
  hipLaunchKernelGGL(route_expand_count_kernel, grid, dim3(256), 0, st, a);
  hipLaunchKernelGGL(route_expand_emit_kernel, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace zha
