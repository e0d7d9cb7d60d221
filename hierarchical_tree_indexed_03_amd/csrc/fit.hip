// Fitting the reference queries to dense attention: the router's training step.
//
// Blog "Zyphra Hierarchical Attention", section "Routing through the tree", and news summary
// "Zyphra releases the ZHA sparse attention method", section "How is ZHA trained onto
// existing models?": the model stays frozen, only the reference queries are trained, and a
// KL loss makes the router's probabilities over the nodes of every level reproduce the
// dense attention mass of those nodes.  For the training queries q of a KV head's group
// (Q of them) and every level l:
//   m_n   = sum over node n's tokens of softmax_t(sigma q.k_t)              (target)
//   pi_n  = softmax over the level of score_n(q) = max_i(sigma q.s_ni + c_ni) (router)
//   loss  = (1/Q) sum_q sum_l KL(m || pi)
// The gradient in r_i runs through the arg-max plane of each (q, node).  Over the node's
// tokens that plane is LSE_i + sigma (q - r_i).s_i, whose derivative in r_i is
// sigma^2 C_i (q - r_i) with C_i the covariance of the node's keys under softmax(sigma r_i.k).
// Summed over nodes and queries, the gradient becomes one weighted sum over the tokens:
//   grad_i   = sigma^2 sum_t alpha_it k_t
//   alpha_it = sum_l w_it (y_itl - beta_il),   w_it = exp(x_it - LSE_i(node of t at level l))
//   y_itl    = (sum_q [i*=i] g_q z_qt - W_i x_it) / sigma        (= k_t.u_i)
//   beta_il  = (sum_q [i*=i] g_q score_q - W_i LSE_i) / sigma    (= s_i.u_i)
// where z_qt = sigma q.k_t, x_it = sigma r_i.k_t, g_q = (pi - m)/Q at the node,
// W_i = sum_q [i*=i] g_q and u_i = sum_q [i*=i] g_q (q - r_i); s_i.q and s_i.r_i come from
// the score (sigma q.s_i + c_i) and from LSE_i = sigma r_i.s_i + c_i, so no d-vector per
// node is ever formed.
//
// Launch sequence (one stream): refs to the cache dtype -> tree build -> sigma*q in fp32 ->
// dense logits z (MFMA) -> node log masses per level -> router scores and arg-max planes per
// level (fp32 MFMA) -> per-row softmax, KL and g -> per-node (W, beta) -> alpha per token ->
// partial gradients per token chunk -> gradient, loss and the SGD update.
#include "common.hpp"
#include "kernels.hpp"
#include "qk_tile.hpp"
#include "route_util.hpp"

namespace zha {

constexpr int FIT_CHUNK = 256;    // tokens per partial-gradient workgroup

__device__ __forceinline__ const float* lse_row(const FitArgs& a, int lv, int kv, int64_t node) {
  return a.dev.lse[lv] + ((int64_t)kv * a.dev.ncap[lv] + node) * a.R;
}

// ------------------------------------------------------------------ inputs
template <typename TIn>
__global__ __launch_bounds__(256) void fit_cast_refs_kernel(FitArgs a) {
  const int64_t n = (int64_t)a.hkv * a.R * a.D;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const float x = a.refs_master[i];
    if constexpr (sizeof(TIn) == 2) {
      const uint32_t bits = f2bf16_bits(x);
      ((bf16_t*)a.refs_in)[i].bits = (uint16_t)bits;
      a.refs_r[i] = bf16_bits_to_f32(bits);
    } else {
      ((float*)a.refs_in)[i] = x;
      a.refs_r[i] = x;
    }
  }
}

// sigma * q in fp32, per KV head in group order: qf[kv][qi][D], qi = batch * g + head.
template <typename TIn>
__global__ __launch_bounds__(256) void fit_prep_q_kernel(FitArgs a) {
  const int64_t n = (int64_t)a.hkv * a.Q * a.D;
  const TIn* q = (const TIn*)a.q;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t d = i % a.D, row = i / a.D;
    const int64_t kv = row / a.Q, qi = row % a.Q;
    const int64_t src = ((qi / a.g) * a.hq + kv * a.g + qi % a.g) * a.D + d;
    a.qf[i] = a.sigma * to_f32(q[src]);
  }
}

// ------------------------------------------------------------------ dense logits
// z[kv][qi][t] = sigma q.k_t for every token: K (16 tokens) . Q^T (16 queries) MFMA tiles;
// a wave keeps its 16 keys and walks the query tiles.
template <typename TIn, int D>
__global__ __launch_bounds__(256) void fit_logits_kernel(FitArgs a) {
  constexpr int NK = Qk<TIn, D>::NL;
  const int kv = blockIdx.y, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, kg = lane >> 4;
  const TIn* Kb = (const TIn*)a.K + (int64_t)kv * a.cap * D;
  const TIn* q = (const TIn*)a.q;
  const int64_t ntile = (a.N + 15) / 16;
  for (int64_t tile = (int64_t)blockIdx.x * 4 + wave; tile < ntile; tile += (int64_t)gridDim.x * 4) {
    const int64_t t0 = tile * 16;
    uint4 kf[NK];
    if (t0 + col < a.N) Qk<TIn, D>::load_k(Kb + (t0 + col) * D, kg, kf);
    else
#pragma unroll
      for (int k = 0; k < NK; ++k) kf[k] = make_uint4(0, 0, 0, 0);
    for (int qt = 0; qt * 16 < a.Q; ++qt) {
      const int qi = qt * 16 + col;
      Qk<TIn, D> qk;
      const TIn* row = qi < a.Q ? q + ((int64_t)(qi / a.g) * a.hq + (int64_t)kv * a.g + qi % a.g) * D : nullptr;
      if constexpr (sizeof(TIn) == 2) {
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
          const uint4 v = row ? *(const uint4*)(row + kg * (D / 4) + kk * 8) : make_uint4(0, 0, 0, 0);
          qk.q[kk] = __builtin_bit_cast(bf16x8, v);
        }
      } else {
#pragma unroll
        for (int i = 0; i < D / 4; ++i) qk.q[i] = row ? row[kg * (D / 4) + i] : 0.f;
      }
      const f32x4 acc = qk.mma(kf);   // acc[e]: token t0 + 4 kg + e, query qi
      if (qi < a.Q) {
        float* zr = a.z + ((int64_t)kv * a.Q + qi) * a.zstride + t0 + 4 * kg;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (t0 + 4 * kg + e < a.N) zr[e] = a.sigma * acc[e];
      }
    }
  }
}

// ------------------------------------------------------------------ dense node mass
// lt[lv][kv][qi][n] = logsumexp of the node's children: the tokens' logits at level 1, the
// child nodes' values above.
__global__ __launch_bounds__(256) void fit_lse_kernel(FitArgs a, int lv) {
  const int64_t nn = a.nl[lv], st = a.nstride[lv];
  const int64_t total = (int64_t)a.hkv * a.Q * nn;
  const int64_t nch = lv == 1 ? a.N : a.nl[lv - 1];
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t n = i % nn, row = i / nn;
    const float* src = lv == 1 ? a.z + row * a.zstride : a.lt[lv - 1] + row * a.nstride[lv - 1];
    const int64_t c0 = n * a.b, c1 = c0 + a.b < nch ? c0 + a.b : nch;
    float mx = -INFINITY;
    for (int64_t c = c0; c < c1; ++c) mx = fmaxf(mx, src[c]);
    float s = 0.f;
    for (int64_t c = c0; c < c1; ++c) s += expf(src[c] - mx);
    a.lt[lv][row * st + n] = mx + logf(s);
  }
}

// ------------------------------------------------------------------ router scores
// score and arg-max plane of every (query, node) of a level: the 16 plane rows of a tile
// (16/R nodes x R planes) against 16 queries at a time on fp32 MFMA, the contraction
// permuted as in the decode's plane scoring (lane (col, kg) streams the 16-byte pieces
// [16 i + 4 kg, +4) of its row); the max over a node's planes runs across R lanes, lowest
// plane on a tie.  The workgroup stages 64 queries at a time in LDS (rows padded by 4
// floats); its four waves then stride over the level's plane tiles against them.
constexpr int FIT_QB = 64;
template <int D, int R>
__global__ __launch_bounds__(256) void fit_score_kernel(FitArgs a, int lv) {
  constexpr int NPT = 16 / R;
  constexpr int NI = D / 16;
  constexpr int QS = D + 4;
  __shared__ __align__(16) float qs[FIT_QB * QS];
  const int kv = blockIdx.y, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, kg = lane >> 4;
  const int slot = col / R, plane = col % R;
  const int64_t nn = a.nl[lv], cap = a.dev.ncap[lv], st = a.nstride[lv];
  const float* S = a.dev.s[lv] + (int64_t)kv * cap * R * D;
  const float* C = a.dev.c[lv] + (int64_t)kv * cap * R;
  const int64_t ntiles = (nn + NPT - 1) / NPT;
  const float* qg = a.qf + (int64_t)kv * a.Q * D;
  for (int qb = 0; qb < a.Q; qb += FIT_QB) {
    __syncthreads();
    for (int i = threadIdx.x; i < FIT_QB * (D / 4); i += 256) {
      const int row = i / (D / 4), c4 = i % (D / 4);
      const float4 v = qb + row < a.Q ? *(const float4*)(qg + (int64_t)(qb + row) * D + 4 * c4)
                                      : make_float4(0.f, 0.f, 0.f, 0.f);
      *(float4*)(qs + row * QS + 4 * c4) = v;
    }
    __syncthreads();
    for (int64_t tile = (int64_t)blockIdx.x * 4 + wave; tile < ntiles; tile += (int64_t)gridDim.x * 4) {
      const int64_t node = tile * NPT + slot;
      const bool ok = node < nn;
      const float* sp = S + ((ok ? node : 0) * R + plane) * D + 4 * kg;
      float4 sb[NI];
#pragma unroll
      for (int i = 0; i < NI; ++i) sb[i] = ok ? *(const float4*)(sp + 16 * i) : make_float4(0.f, 0.f, 0.f, 0.f);
      const float cj = ok ? C[node * R + plane] : -INFINITY;
      for (int qt = 0; qt < FIT_QB / 16 && qb + qt * 16 < a.Q; ++qt) {
        const float* qp = qs + (qt * 16 + col) * QS + 4 * kg;   // A operand row of this lane
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const float4 qv = *(const float4*)(qp + 16 * i);
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qv.x, sb[i].x, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qv.y, sb[i].y, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qv.z, sb[i].z, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qv.w, sb[i].w, acc, 0, 0, 0);
        }
        // acc[e]: query qb + qt*16 + 4 kg + e, plane row col
        float v[4];
        int im[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) { v[e] = acc[e] + cj; im[e] = plane; }
#pragma unroll
        for (int off = 1; off < R; off <<= 1)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float ov = __shfl_xor(v[e], off);
            const int oi = __shfl_xor(im[e], off);
            if (ov > v[e] || (ov == v[e] && oi < im[e])) { v[e] = ov; im[e] = oi; }
          }
        if (ok && plane == 0) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int qi = qb + qt * 16 + 4 * kg + e;
            if (qi < a.Q) {
              const int64_t o = ((int64_t)kv * a.Q + qi) * st + node;
              a.sc[lv][o] = v[e];
              a.am[lv][o] = (uint8_t)im[e];
            }
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------------ loss and d loss / d score
__device__ __forceinline__ float block_max256(float v, float* red) {
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}
__device__ __forceinline__ float block_sum256(float v, float* red) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// One workgroup per (query, level, KV head): m and pi over the level's nodes, KL(m || pi)
// and g = (pi - m) / Q.
__global__ __launch_bounds__(256) void fit_loss_kernel(FitArgs a) {
  __shared__ float red[4];
  const int qi = blockIdx.x, lv = blockIdx.y + 1, kv = blockIdx.z;
  const int64_t nn = a.nl[lv];
  const int64_t o = ((int64_t)kv * a.Q + qi) * a.nstride[lv];
  const float* sc = a.sc[lv] + o;
  const float* lt = a.lt[lv] + o;
  float* gr = a.gr[lv] + o;
  float ms = -INFINITY, ml = -INFINITY;
  for (int64_t n = threadIdx.x; n < nn; n += 256) { ms = fmaxf(ms, sc[n]); ml = fmaxf(ml, lt[n]); }
  ms = block_max256(ms, red);
  ml = block_max256(ml, red);
  float ss = 0.f, sl = 0.f;
  for (int64_t n = threadIdx.x; n < nn; n += 256) { ss += expf(sc[n] - ms); sl += expf(lt[n] - ml); }
  ss = block_sum256(ss, red);
  sl = block_sum256(sl, red);
  const float lse_s = ms + logf(ss), lse_l = ml + logf(sl);
  const float invq = 1.0f / (float)a.Q;
  float kl = 0.f;
  for (int64_t n = threadIdx.x; n < nn; n += 256) {
    const float logpi = sc[n] - lse_s, logm = lt[n] - lse_l;
    const float m = expf(logm);
    if (m > 0.f) kl += m * (logm - logpi);
    gr[n] = (expf(logpi) - m) * invq;
  }
  kl = block_sum256(kl, red);
  if (threadIdx.x == 0) a.kl[((int64_t)kv * a.Q + qi) * a.levels + (lv - 1)] = kl;
}

// ------------------------------------------------------------------ per-node sums
// wb[lv][kv][n][i] = (W_i, beta_i): W_i = sum of g over the queries whose arg-max plane at
// the node is i, beta_i = (sum of g * score over them - W_i LSE_i) / sigma.  One wave per
// node: lane l takes queries l, l + 64, ...; the per-plane sums are reduced across the wave
// in a fixed order.
template <int R>
__global__ __launch_bounds__(256) void fit_node_kernel(FitArgs a, int lv) {
  const int lane = threadIdx.x & 63;
  const int64_t nn = a.nl[lv], st = a.nstride[lv];
  const int64_t total = (int64_t)a.hkv * nn;
  for (int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); i < total; i += (int64_t)gridDim.x * 4) {
    const int kv = (int)(i / nn);
    const int64_t n = i % nn;
    float W[R], B[R];
#pragma unroll
    for (int r = 0; r < R; ++r) { W[r] = 0.f; B[r] = 0.f; }
    for (int qi = lane; qi < a.Q; qi += 64) {
      const int64_t o = ((int64_t)kv * a.Q + qi) * st + n;
      const int p = a.am[lv][o];
      const float g = a.gr[lv][o], s = a.sc[lv][o];
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (p == r) { W[r] += g; B[r] += g * s; }
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
      for (int off = 32; off > 0; off >>= 1) {
        W[r] += __shfl_xor(W[r], off);
        B[r] += __shfl_xor(B[r], off);
      }
    if (lane < R) {
      float w = 0.f, bsum = 0.f;
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (lane == r) { w = W[r]; bsum = B[r]; }
      const float L = lse_row(a, lv, kv, n)[lane];
      ((float2*)a.wb[lv])[((int64_t)kv * st + n) * R + lane] = make_float2(w, (bsum - w * L) / a.sigma);
    }
  }
}

// ------------------------------------------------------------------ alpha per token
// alpha[kv][t][i] = sum over levels of w_it (y_itl - beta_il) (see the top of the file).
// One thread per token; the (rounded) reference queries sit in LDS.
template <typename TIn, int D, int R>
__global__ __launch_bounds__(256) void fit_alpha_kernel(FitArgs a) {
  __shared__ float rs[R * D];
  const int kv = blockIdx.y;
  for (int i = threadIdx.x; i < R * D; i += 256) rs[i] = a.refs_r[(int64_t)kv * R * D + i];
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= a.N) return;
  const TIn* kr = (const TIn*)a.K + ((int64_t)kv * a.cap + t) * D;
  float x[R];
#pragma unroll
  for (int r = 0; r < R; ++r) x[r] = 0.f;
  for (int d0 = 0; d0 < D; d0 += 8) {
    float k8[8];
    if constexpr (sizeof(TIn) == 2) {
      const uint4 w = *(const uint4*)(kr + d0);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) { k8[2 * j] = bf16_bits_to_f32(ww[j] & 0xffffu); k8[2 * j + 1] = bf16_bits_to_f32(ww[j] >> 16); }
    } else {
      const float4 u = *(const float4*)((const float*)kr + d0);
      const float4 v = *(const float4*)((const float*)kr + d0 + 4);
      k8[0] = u.x; k8[1] = u.y; k8[2] = u.z; k8[3] = u.w; k8[4] = v.x; k8[5] = v.y; k8[6] = v.z; k8[7] = v.w;
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int j = 0; j < 8; ++j) x[r] += rs[r * D + d0 + j] * k8[j];
  }
#pragma unroll
  for (int r = 0; r < R; ++r) x[r] *= a.sigma;
  float al[R];
#pragma unroll
  for (int r = 0; r < R; ++r) al[r] = 0.f;
  int64_t span = 1;
  for (int lv = 1; lv <= a.levels; ++lv) {
    span *= a.b;
    const int64_t n = t / span, st = a.nstride[lv];
    float Y[R];
#pragma unroll
    for (int r = 0; r < R; ++r) Y[r] = 0.f;
#pragma unroll 4
    for (int qi = 0; qi < a.Q; ++qi) {
      const int64_t o = ((int64_t)kv * a.Q + qi) * st + n;
      const int p = a.am[lv][o];
      const float cz = a.gr[lv][o] * a.z[((int64_t)kv * a.Q + qi) * a.zstride + t];
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (p == r) Y[r] += cz;
    }
    const float* L = lse_row(a, lv, kv, n);
    const float2* wb = (const float2*)a.wb[lv] + ((int64_t)kv * st + n) * R;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float2 v = wb[r];
      const float y = (Y[r] - v.x * x[r]) / a.sigma;
      al[r] += expf(x[r] - L[r]) * (y - v.y);
    }
  }
  float* out = a.alpha + ((int64_t)kv * a.N + t) * R;
#pragma unroll
  for (int r = 0; r < R; ++r) out[r] = al[r];
}

// ------------------------------------------------------------------ gradient
// part[kv][chunk][i][d] = sum over the chunk's tokens of alpha_it k_t[d]: 256 threads = D
// dimensions x 256/D token groups, the groups summed through LDS in a fixed order.
template <typename TIn, int D, int R>
__global__ __launch_bounds__(256) void fit_grad_kernel(FitArgs a) {
  constexpr int TG = 256 / D;
  __shared__ float red[TG][R][D];
  const int kv = blockIdx.y, chunk = blockIdx.x;
  const int d = threadIdx.x % D, tg = threadIdx.x / D;
  const int64_t t0 = (int64_t)chunk * FIT_CHUNK;
  const int64_t t1 = t0 + FIT_CHUNK < a.N ? t0 + FIT_CHUNK : a.N;
  const TIn* Kb = (const TIn*)a.K + (int64_t)kv * a.cap * D;
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.f;
#pragma unroll 4
  for (int64_t t = t0 + tg; t < t1; t += TG) {
    const float k = to_f32(Kb[t * D + d]);
    const float* al = a.alpha + ((int64_t)kv * a.N + t) * R;
    if constexpr (R % 4 == 0) {
#pragma unroll
      for (int r = 0; r < R; r += 4) {
        const float4 v = *(const float4*)(al + r);
        acc[r] += v.x * k; acc[r + 1] += v.y * k; acc[r + 2] += v.z * k; acc[r + 3] += v.w * k;
      }
    } else {
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] += al[r] * k;
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) red[tg][r][d] = acc[r];
  __syncthreads();
  float* out = a.part + ((int64_t)kv * a.nchunk + chunk) * R * D;
  for (int i = threadIdx.x; i < R * D; i += 256) {
    float sum = 0.f;
#pragma unroll
    for (int g2 = 0; g2 < TG; ++g2) sum += red[g2][i / D][i % D];
    out[i] = sum;
  }
}

// grad = sigma^2 * (sum of the partials, in chunk order); loss = sum of the KL rows / Q;
// refs -= lr * grad.  One thread per gradient element (grid x over R*D/256, y over KV heads).
__global__ __launch_bounds__(256) void fit_update_kernel(FitArgs a) {
  const int kv = blockIdx.y;
  const int64_t nrd = (int64_t)a.R * a.D;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < nrd) {
    const float* p = a.part + (int64_t)kv * a.nchunk * nrd + i;
    float sum = 0.f;
#pragma unroll 8
    for (int c = 0; c < a.nchunk; ++c) sum += p[(int64_t)c * nrd];
    const float g = a.sigma * a.sigma * sum;
    a.grad[(int64_t)kv * nrd + i] = g;
    if (a.lr != 0.f) a.refs_master[(int64_t)kv * nrd + i] -= a.lr * g;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    float l = 0.f;
    for (int64_t j = 0; j < (int64_t)a.Q * a.levels; ++j) l += a.kl[(int64_t)kv * a.Q * a.levels + j];
    a.loss[kv] = l / (float)a.Q;
  }
}

// ------------------------------------------------------------------ launchers
static unsigned grid_n(int64_t n, int per) { return grid_for(n, per, 1 << 16); }

template <typename TIn, int D, int R>
static hipError_t fit_stage_t(const FitArgs& a, int stage, hipStream_t st) {
  switch (stage) {
    case FIT_LOGITS: {
      hipLaunchKernelGGL(fit_prep_q_kernel<TIn>, dim3(grid_n((int64_t)a.hkv * a.Q * D, 256)), dim3(256), 0, st, a);
      const int64_t ntile = (a.N + 15) / 16;
      hipLaunchKernelGGL((fit_logits_kernel<TIn, D>), dim3(grid_for(ntile, 4, 2048), (unsigned)a.hkv), dim3(256), 0, st, a);
      break;
    }
    case FIT_MASS:
      for (int lv = 1; lv <= a.levels; ++lv)
        hipLaunchKernelGGL(fit_lse_kernel, dim3(grid_n((int64_t)a.hkv * a.Q * a.nl[lv], 256)), dim3(256), 0, st, a, lv);
      break;
    case FIT_SCORE:
      for (int lv = 1; lv <= a.levels; ++lv) {
        const int64_t ntiles = (a.nl[lv] + 16 / R - 1) / (16 / R);
        static const int per_cu = resident_per_cu(fit_score_kernel<D, R>, 256);
        const int64_t cap = (int64_t)per_cu * device_cus() / a.hkv;
        hipLaunchKernelGGL((fit_score_kernel<D, R>), dim3(grid_for(ntiles, 4, cap), (unsigned)a.hkv), dim3(256), 0, st, a, lv);
      }
      break;
    case FIT_LOSS:
      hipLaunchKernelGGL(fit_loss_kernel, dim3((unsigned)a.Q, (unsigned)a.levels, (unsigned)a.hkv), dim3(256), 0, st, a);
      for (int lv = 1; lv <= a.levels; ++lv)
        hipLaunchKernelGGL((fit_node_kernel<R>), dim3(grid_n((int64_t)a.hkv * a.nl[lv], 4)), dim3(256), 0, st, a, lv);
      break;
    case FIT_ALPHA:
      hipLaunchKernelGGL((fit_alpha_kernel<TIn, D, R>), dim3((unsigned)((a.N + 255) / 256), (unsigned)a.hkv), dim3(256), 0, st, a);
      break;
    case FIT_GRAD:
      hipLaunchKernelGGL((fit_grad_kernel<TIn, D, R>), dim3((unsigned)a.nchunk, (unsigned)a.hkv), dim3(256), 0, st, a);
      hipLaunchKernelGGL(fit_update_kernel, dim3((unsigned)((R * D + 255) / 256), (unsigned)a.hkv), dim3(256), 0, st, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_fit_cast_refs(const FitArgs& a, bool bf16, hipStream_t st) {
  const unsigned grid = grid_n((int64_t)a.hkv * a.R * a.D, 256);
  if (bf16) hipLaunchKernelGGL(fit_cast_refs_kernel<bf16_t>, dim3(grid), dim3(256), 0, st, a);
  else hipLaunchKernelGGL(fit_cast_refs_kernel<float>, dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_fit_stage(const FitArgs& a, bool bf16, int stage, hipStream_t st) {
#define ZHA_CASE(DD, RR)                                                              \
  if (a.D == DD && a.R == RR)                                                         \
    return bf16 ? fit_stage_t<bf16_t, DD, RR>(a, stage, st) : fit_stage_t<float, DD, RR>(a, stage, st);
  ZHA_CASE(64, 1) ZHA_CASE(64, 2) ZHA_CASE(64, 4) ZHA_CASE(64, 8) ZHA_CASE(64, 16)
  ZHA_CASE(128, 1) ZHA_CASE(128, 2) ZHA_CASE(128, 4) ZHA_CASE(128, 8) ZHA_CASE(128, 16)
#undef ZHA_CASE
  return hipErrorInvalidValue;
}

int fit_chunk_tokens() { return FIT_CHUNK; }

}  // namespace zha
