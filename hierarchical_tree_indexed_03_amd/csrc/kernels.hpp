// Kernel argument blocks and host-side launchers of the ZHA HIP library.
#pragma once
#include "common.hpp"

namespace zha {

struct BuildArgs {
  const void* K;      // [Hkv][cap][D]
  const void* refs;   // [Hkv][R][D]
  int64_t cap;
  int64_t N;
  int32_t b;
  int32_t m;          // levels built inside one tile
  float sigma;
  int64_t tile0;      // first tile to build (0: the whole tree)
  Dev dev;
};

struct ParentArgs {
  Dev dev;
  int32_t level;      // level being built (>= 2)
  int32_t b;
  int64_t nparent;    // nodes at `level`
  int64_t nchild;     // nodes at `level - 1`
  int64_t first;      // first parent to build (0: the whole level)
};

struct QuantArgs {
  Dev dev;
  int32_t level;
  int64_t first;      // nodes first .. nnode-1 of the level are quantised
  int64_t nnode;
};

struct AppendArgs {
  void* K;
  void* V;
  const void* k_new;  // row of KV head kv at k_new + kv * new_stride elements
  const void* v_new;
  int64_t new_stride; // elements between the KV heads' rows (D for a [Hkv][D] token)
  const void* refs;
  int64_t cap;
  int64_t N;          // index of the new token (tokens before the append)
  int32_t b;
  int32_t levels;
  float sigma;
  Dev dev;
};

struct RouteArgs {
  Dev dev;
  const void* q;      // [Hq][D] input dtype
  int64_t N;          // tokens
  int32_t hkv, hq, g, b, levels;
  int32_t level;      // level being routed
  int64_t nlevel;     // nodes at `level` (upper bound of every union frontier there)
  int64_t nbelow;     // nodes at level-1 (children existence); unused at level 1
  float sigma;
  float top_p[MAXL + 1];  // p of the top-p decision at each level (index = level)
  int32_t dense;      // score kernel: 1 = every node of levels `level` .. `level`-gridDim.z+1
  int32_t dense_lo;   // lowest level handled by the multi-level selection kernel
  int32_t tf;         // top-down selection: the top level's per-head frontier is given in
                      // dev.tdbits (teacher forcing) instead of being every node
  int32_t sel_p;      // top-p histogram / classify workgroups per KV head at `level`
  int32_t key_form;   // level 1 scored from the block's keys and the planes' token weights
  int32_t nref;       // reference queries (planes per node)
  int32_t allkeys;    // every level scored from the keys (route_score_allkeys_kernel) and
                      // selected top-down with level 1 (route_topdown_keys_kernel)
  int32_t prep_fold;  // route_score_allkeys_kernel also does the route prep's part of that path
                      // (list sizes, arrival counts): the decode then launches no prep kernel
  int32_t q_bf16;     // q (and the caches) are bf16; else fp32
  int32_t planes;     // router planes read: 0 fp32 (dev.s), 1 bf16 (dev.sq), 2 MX FP4 (dev.s4, dev.s4x)
  const void* K;      // key cache [Hkv][kcap][D] (key-form scoring)
  int64_t kcap;
  int64_t nl[MAXL + 1];   // nodes per level at N
};

// Top-down bitmaps of query head hq at level lv: frontier words, then (td_stride words
// later) kept words.
__device__ __forceinline__ int64_t td_stride(const RouteArgs& a, int lv) {
  return (lv == 1 && a.allkeys) ? a.dev.ncap[1] / 32 : (int64_t)TD_WORDS;
}
__device__ __forceinline__ uint32_t* td_front_words(const RouteArgs& a, int lv, int hq) {
  if (lv == 1 && a.allkeys) return a.dev.kb1 + (int64_t)hq * 2 * (a.dev.ncap[1] / 32);
  return a.dev.tdbits + (((int64_t)lv * a.hq + hq) * 2) * TD_WORDS;
}
__device__ __forceinline__ uint32_t* td_kept_words(const RouteArgs& a, int lv, int hq) {
  return td_front_words(a, lv, hq) + td_stride(a, lv);
}

struct AttnArgs {
  Dev dev;
  const void* K;
  const void* V;
  const void* q;
  int64_t cap;
  int64_t N;
  int32_t hkv, hq, g, b;
  int32_t splits;     // splits per KV head (grid.x)
  int32_t pstride;    // partials per query head in dev.apart ([Hq][pstride][D + 2]), >= splits
  int32_t keep_sink;
  float sigma;
  float* out;         // [Hq][D]
  // several queries in one routed launch (grid.y = query; a decode has one and zero strides):
  // query y reads q + y * q_stride, its gather list at dev.node[0] / dev.mask[0] +
  // y * l_stride and its counts at dev.cnt + y * c_stride, attends tokens below
  // N + y * n_step, and writes its partials at dev.apart + y * p_stride and its output at
  // out + y * o_stride
  int64_t q_stride, l_stride, p_stride, o_stride;
  int32_t c_stride, n_step;
};

// Batched causal prefill (prefill.hip): mb queries at positions N0 .. N0 + mb - 1, query i
// routed over the tree of tokens [0, N0 + i]; pair p = i * g + gi is query i's head gi.
struct PrefillArgs {
  Dev dev;
  const void* K;          // [Hkv][cap][D] cache dtype
  const void* refs;       // [Hkv][R][D]
  const void* q;          // [mb][Hq][D] cache dtype (this sub-batch)
  const void* V;          // [Hkv][cap][D] cache dtype
  int32_t keep_sink;
  int64_t cap;
  int64_t N0;             // tokens before the sub-batch
  int32_t mb, mbmax, P, hkv, hq, g, b, levels, R, D;
  int32_t q_bf16;
  float sigma;
  float top_p[MAXL + 1];
  int64_t nl[MAXL + 1];   // nodes per level of the tree over N0 + mb tokens
  float* Qf;              // [Hkv][P][D] sigma * q in fp32
  float* X;               // [Hkv][mbmax][levels + 1][R][D + 2] per query and level: its rightmost node
                          // (s, c, LSE per plane) over the tokens up to its own
  float* S;               // scores, level l at S + soff[l]: [Hkv][P][sstride[l]]
  int64_t soff[MAXL + 1], sstride[MAXL + 1];
  uint32_t* KB;           // kept bitmaps, level l at KB + koff[l]: [Hkv][P][kstride[l]] words
  int64_t koff[MAXL + 1], kstride[MAXL + 1];
  int32_t* L0node;        // [mbmax][Hkv][ncap1] gather list of each query (kept level-1 blocks)
  uint32_t* L0mask;       // the heads of the query that kept each block
  int32_t* cnt0;          // [mbmax][Hkv]
};
hipError_t launch_prefill_prefix(const PrefillArgs& a, bool bf16, int D, int R, hipStream_t st);
hipError_t launch_prefill_qprep(const PrefillArgs& a, bool bf16, int D, hipStream_t st);
hipError_t launch_prefill_score(const PrefillArgs& a, int D, int R, hipStream_t st);
hipError_t launch_prefill_tail(const PrefillArgs& a, int D, int R, hipStream_t st);
hipError_t launch_prefill_select(const PrefillArgs& a, hipStream_t st);
hipError_t launch_prefill_gather(const PrefillArgs& a, hipStream_t st);
// Union attention of a sub-batch (bf16 caches): partials [Hkv][P][splits][D + 2] in `part`,
// then the merged output of query i, head h at out + (i * Hq + h) * D.
int prefill_attend_splits(int hkv, int P);
hipError_t launch_prefill_attend(const PrefillArgs& a, float* part, float* out, int D, hipStream_t st);
// Routed attention and combine for a.nq... queries of one launch (grid.y = query).
hipError_t launch_attend_batch(const AttnArgs& a, bool bf16, int D, int nq, hipStream_t st);

// One fitting step of the reference queries (fit.hip): buffers in the caller's fit
// workspace, the tree's planes and log masses in dev.
struct FitArgs {
  Dev dev;
  const void* K;          // [Hkv][cap][D] cache dtype
  const void* q;          // [nq][Hq][D] cache dtype: the training queries
  float* refs_master;     // [Hkv][R][D] float32 reference queries (the SGD update writes here)
  void* refs_in;          // [Hkv][R][D] cache dtype: their rounding, which the tree is built from
  float* refs_r;          // [Hkv][R][D] float32 values of refs_in
  float* qf;              // [Hkv][Q][D] sigma * q, group order (qi = batch * g + head)
  float* z;               // [Hkv][Q][zstride] dense logits sigma q.k_t
  float* lt[MAXL + 1];    // [Hkv][Q][nstride[l]] logsumexp of the logits over each node
  float* sc[MAXL + 1];    // router score of each node
  float* gr[MAXL + 1];    // d loss / d score = (pi - m) / Q
  uint8_t* am[MAXL + 1];  // arg-max plane of each score
  float* wb[MAXL + 1];    // [Hkv][nstride[l]][R][2] per node and plane: W and beta
  float* kl;              // [Hkv][Q][levels] KL(m || pi) per query and level
  float* alpha;           // [Hkv][N][R]
  float* part;            // [Hkv][nchunk][R][D] partial gradients
  float* grad;            // [Hkv][R][D]
  float* loss;            // [Hkv]
  int64_t cap, N, zstride;
  int64_t nl[MAXL + 1];       // nodes per level at N
  int64_t nstride[MAXL + 1];  // row stride of the per-level arrays (nl rounded up to 64)
  int32_t hkv, hq, g, Q, b, levels, R, D, nchunk;
  float sigma, lr;
};

// The fitting step after the tree build, stage by stage (in this order): dense logits,
// dense node log masses, router scores, loss and per-node sums, alpha per token, gradient
// and update.
enum FitStage { FIT_LOGITS = 0, FIT_MASS, FIT_SCORE, FIT_LOSS, FIT_ALPHA, FIT_GRAD, FIT_NSTAGE };
hipError_t launch_fit_cast_refs(const FitArgs& a, bool bf16, hipStream_t st);
hipError_t launch_fit_stage(const FitArgs& a, bool bf16, int stage, hipStream_t st);
int fit_chunk_tokens();

hipError_t launch_build_tile(const BuildArgs& a, bool bf16, int D, int R, int64_t ntiles, int hkv, int T,
                             hipStream_t st);
hipError_t launch_build_parent(const ParentArgs& a, int D, int R, int hkv, hipStream_t st);
// Levels 1 and 2 (a.m = 1 or 2) for R <= 4 and b in {2, 4, 8}, keys held in registers;
// tiles of narrow_tile_tokens(D, b) tokens.
bool narrow_build(int R, int b);
int narrow_tile_tokens(int D, int b);
hipError_t launch_build_narrow(const BuildArgs& a, bool bf16, int D, int R, int hkv, hipStream_t st);
hipError_t launch_append(const AppendArgs& a, bool bf16, int D, int R, int hkv, hipStream_t st);
// MX FP4 router copies (dev.s4, dev.s4x) of one level's float32 s.
hipError_t launch_quantise_fp4(const QuantArgs& a, int D, int R, int hkv, hipStream_t st);

// Routing: prep (q to fp32, state reset, top frontier) then per level the step sequence.
hipError_t launch_route_prep(const RouteArgs& a, bool bf16, int D, hipStream_t st);
hipError_t launch_route_score(const RouteArgs& a, int D, int R, hipStream_t st);
hipError_t launch_route_select(const RouteArgs& a, hipStream_t st);   // hist, bound, classify, resolve
hipError_t launch_route_expand(const RouteArgs& a, hipStream_t st);
// Top levels with at most TD_MAX nodes: score every node of levels `level`..`dense_lo` in
// one launch, then select all of them top-down (one workgroup per query head).
hipError_t launch_route_dense_score(const RouteArgs& a, int D, int R, hipStream_t st);
hipError_t launch_route_topdown(const RouteArgs& a, hipStream_t st);
// Dense union lists (node, frontier mask, keep mask) of the top-down levels
// a.dense_lo .. a.level from the top-down bitmaps.
hipError_t launch_route_td_lists(const RouteArgs& a, hipStream_t st);
// The dense union list of level a.dense_lo - 1 (masks = the heads that kept each parent),
// from the top-down kept bitmaps of level a.dense_lo (a.dense_lo >= 2).
hipError_t launch_route_td_children(const RouteArgs& a, hipStream_t st);
// Per-head frontier bitmaps of level a.level in dev.tdbits from that level's union list
// (dev.node / dev.mask / dev.cnt): the given frontier of a teacher-forced top-down level.
hipError_t launch_route_td_seed(const RouteArgs& a, hipStream_t st);
// Every level from the keys (a.allkeys): scores of levels 1..4 and the level-4 dot products
// in one pass over the key cache; then the levels above level 4 derived, and every level
// from a.level down to a.dense_lo selected top-down (one workgroup per query head); then the
// gather list of the kept level-1 blocks per KV head.
hipError_t launch_route_allkeys_score(const RouteArgs& a, int D, int R, hipStream_t st);
hipError_t launch_route_topdown_keys(const RouteArgs& a, hipStream_t st);

hipError_t launch_attend(const AttnArgs& a, bool bf16, int D, bool dense, hipStream_t st);
// Attention workgroups resident on the GPU at once, per KV head (one wave of workgroups).
int attend_resident_splits(bool bf16, int D, bool dense, int hkv);
// Same, and copies the per-level union sizes into `stats` ([levels + 1][Hkv], nullable).
hipError_t launch_attend_full(const AttnArgs& a, bool bf16, int D, bool dense, int32_t* stats, int levels,
                              hipStream_t st);

}  // namespace zha
