/*
 * zha.h — C ABI of the ZHA (Zyphra Hierarchical Attention) decode hot path on MI355X.
 *
 * The method (arXiv 2610.42112, "Subquadratic Attention with a Hierarchical
 * Tree-Structured Indexer"; Zyphra blog post "Zyphra Hierarchical Attention"):
 *   - the full KV cache is kept; over its keys a tree of summaries is built: keys are cut
 *     into contiguous blocks of `block` tokens and each block is summarised, then the
 *     summaries are grouped `block` at a time and summarised again, `levels` times
 *     (blog, "Building the tree");
 *   - a summary is, for each of `num_ref` reference queries r_j, a tangent plane of the
 *     node's log attention mass: a weighted-mean key s_j and an offset c_j; a query q
 *     scores the node with max_j(q.s_j/sqrt(d) + c_j) (news summary, "Building the tree");
 *   - a decode query scores the top level, keeps the smallest set of nodes holding a
 *     fraction `top_p` of the estimated attention probability, expands only their children
 *     and repeats down to the raw keys, then runs ordinary attention over the selected
 *     blocks plus token 0, the attention sink (blog, "Routing through the tree"; news
 *     summary, "How does top-p routing pick tokens?").
 *
 * Conventions shared by every call:
 *   - Pointers marked (device) are HIP device memory; (host) are host memory.  The caller
 *     owns every buffer.  The library never allocates or frees device memory and never
 *     synchronises a stream, except where a call says so.
 *   - Tensors are dense, row-major, with the shapes given.  `dtype` (zha_dtype) fixes the
 *     element type of K, V, reference queries and decode queries: float32 or bfloat16.
 *     Tree planes and outputs are float32 (plus optional bfloat16 router copies of s,
 *     see zha_config.plane_dtype).
 *   - Every call validates its arguments on the host before enqueueing any work; on any
 *     error it returns a non-zero zha_status, enqueues nothing and leaves the handle
 *     unchanged.  zha_last_error() then describes the failure (thread-local string).
 *   - Work is asynchronous on the given stream (0 = the null stream).  Faults inside
 *     kernels surface at the caller's next synchronisation.  A handle is not thread-safe.
 *   - Query head h reads KV head h / (num_q_heads / num_kv_heads) (contiguous groups).
 */
#ifndef ZHA_H
#define ZHA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ZHA_OK = 0,
  ZHA_E_INVALID = 1,      /* bad argument: null pointer, out-of-range value        */
  ZHA_E_UNSUPPORTED = 2,  /* valid but not built: head_dim, num_ref or group size   */
  ZHA_E_CAPACITY = 3,     /* token count above the configured capacity             */
  ZHA_E_WORKSPACE = 4,    /* workspace smaller than zha_workspace_bytes()          */
  ZHA_E_STATE = 5,        /* call out of order (e.g. decode before build)          */
  ZHA_E_HIP = 6           /* a HIP runtime call failed; see zha_last_error()       */
} zha_status;

typedef enum { ZHA_F32 = 0, ZHA_BF16 = 1, ZHA_MXFP4 = 2 /* router planes only */ } zha_dtype;

typedef struct {
  int32_t head_dim;       /* d: 64 or 128                                               */
  int32_t num_kv_heads;   /* Hkv >= 1: one tree per KV head                             */
  int32_t num_q_heads;    /* Hq: a multiple of Hkv with Hq/Hkv <= 8                     */
  int32_t block;          /* b: tokens per leaf block / children per node, a power of
                             two in 2..256 (others: ZHA_E_UNSUPPORTED)                  */
  int32_t levels;         /* L: 1..16 summary levels                                    */
  int32_t num_ref;        /* R: 1, 2, 4, 8 or 16 reference queries per tree             */
  int64_t capacity;       /* max tokens the caches (and the tree) may hold              */
  int32_t dtype;          /* zha_dtype of K, V, reference and decode queries            */
  float top_p;            /* p in (0, 1]; p = 1 keeps every node (dense attention)     */
  int32_t keep_sink;      /* 1: token 0 is always attended                              */
  int32_t plane_dtype;    /* zha_dtype of the s vectors the router reads (0 = float32).
                           * The tree is always built and kept in float32; with ZHA_BF16 or
                           * ZHA_MXFP4 each plane the router scores from also gets a
                           * quantised copy of s, and routing reads that copy with the
                           * float32 offset c_j.  The pages give no storage precision for
                           * the planes; these are stated quantisers:
                           *   ZHA_BF16: each element the nearest bfloat16 (ties to even);
                           *     R*(2d+4) bytes per node instead of R*(4d+4);
                           *   ZHA_MXFP4: OCP MX FP4, per 32 elements one power-of-two
                           *     scale X = 2^(floor(log2 amax) - 2) (one E8M0 byte) and
                           *     E2M1 elements (nearest of X*{0,.5,1,1.5,2,3,4,6}, ties to
                           *     the even code, clamped at 6X); R*(d/2+d/32+4) bytes.
                           * A level 1 scored from the keys (see zha_level1_key_form)
                           * reads no planes and keeps no copy.                           */
} zha_config;

typedef struct zha_tree zha_tree;   /* opaque host-side handle */

/* Device workspace needed by a handle: the tree planes at capacity (per level l,
 * s [Hkv][ceil(capacity/b^l)][R][d] and c [Hkv][...][R], float32) plus router and
 * attention scratch.  Returns 0 for an invalid or unsupported config. */
size_t zha_workspace_bytes(const zha_config* cfg);

/* How level 1 is scored for this config (news summary, "Building the tree": a level-1
 * plane's s_j is the softmax-weighted mean of its block's keys, so q.s_j is the same weighted
 * sum of the block's logits q.k_t).  Returns 1 when the library scores level 1 from the
 * block's keys and the stored R x b token weights (bf16 keys, b in {2, 4, 8, 16}, and fewer
 * bytes than the R planes), 0 when it reads the planes, -1 for an invalid config.  Host
 * only; no side effects. */
int32_t zha_level1_key_form(const zha_config* cfg);

/* Whether decode scores EVERY level from the keys for this config by default: 1 yes, 0 no,
 * -1 invalid config.  A node's plane s_j is its children's s_j weighted by
 * exp(LSE_cj - LSE_j) down to the keys (news summary, "Building the tree"; blog, "Building
 * the tree": summaries grouped and compressed again), so q.s_j / sqrt(d) is the same
 * weighted sum of the children's dot products, and every level's scores follow from one
 * pass over the keys, the level-1 token weights and each node's (c_j, LSE_j): d*2 + R*4
 * bytes per token plus 8R per node of levels 1..4, the levels above derived from level 4.
 * Possible for bf16 keys, block 4, at least 4 levels, R in {4, 8, 16}, a level 1 scored
 * from the keys (zha_level1_key_form) and at most 131,072 level-1 nodes at capacity (with
 * levels 2.. at most 33,792 nodes and the levels above level 4 small enough for the
 * selection's on-chip buffers).  Chosen by default when it reads no more bytes than the
 * router planes of levels 2..L plus a level 1 scored whole from the keys.  Every level is
 * then selected top-down, level 1 included, with the same top-p rule.  Host only. */
int32_t zha_route_keys(const zha_config* cfg);

/* Creates a handle over a caller-owned device `workspace` (>= zha_workspace_bytes,
 * 256-byte aligned).  The workspace is borrowed until zha_destroy. */
zha_status zha_create(const zha_config* cfg, void* workspace, size_t workspace_bytes,
                      zha_tree** out);

/* Builds the whole tree over keys [0, n_tokens) (blog, "Building the tree").
 *   k_cache, v_cache  (device) [Hkv][capacity][d] dtype; borrowed until the next build
 *                     or destroy (append writes row N into them; decode reads them).
 *   n_tokens          1..capacity tokens already in the caches.
 *   ref_queries       (device) [Hkv][R][d] dtype; borrowed likewise.
 * Level 1: for block n and reference query r_j, z_t = r_j.k_t/sqrt(d) over the block's
 * keys, LSE = logsumexp z, s_j = sum_t softmax(z)_t k_t, c_j = LSE - r_j.s_j/sqrt(d).
 * Level l > 1: LSE_j = logsumexp over children of their log mass at r_j; s_j = the
 * children's s_j weighted by softmax of those log masses; c_j as above. */
zha_status zha_tree_build(zha_tree* t, void* k_cache, void* v_cache, int64_t n_tokens,
                          const void* ref_queries, hipStream_t stream);

/* Appends m >= 1 tokens to every KV head at once (a prompt chunk, or tokens accepted
 * together): copies k_new/v_new ((device) [Hkv][m][d] dtype) into rows N..N+m-1 of the
 * caches, then rebuilds every node whose span holds one of them: the key tiles from the
 * one holding row N, and at each level the nodes from the one holding row N (the same
 * kernels as zha_tree_build, so the result equals a build over N+m tokens).  Cost grows
 * with m plus one tile and one node per level.  ZHA_E_CAPACITY when N + m > capacity.
 * The pages state the tree is built over the KV cache and grows with it (blog,
 * "Building the tree"); bulk growth is the build restricted to the new tail. */
zha_status zha_tree_append_n(zha_tree* t, const void* k_new, const void* v_new, int64_t m,
                             hipStream_t stream);

/* Appends one token to every KV head: writes k_new/v_new ((device) [Hkv][d] dtype) into
 * row N of the caches, then refreshes the one node per level whose span holds the new
 * token.  ZHA_E_CAPACITY when N == capacity.  Equivalent to a rebuild over N+1 tokens. */
zha_status zha_tree_append(zha_tree* t, const void* k_new, const void* v_new,
                           hipStream_t stream);

/* Fitting the reference queries (blog, "Routing through the tree"; news summary, "How is
 * ZHA trained onto existing models?": the model stays frozen, only the reference queries
 * are trained, and a KL loss matches the router's probabilities to the dense attention
 * mass of every node at every level).  One call is one step of gradient descent on
 *   loss_kv = (1/Q) sum over the Q = nq * (Hq/Hkv) training queries of the KV head's group
 *             sum over levels l of KL(m_l || pi_l),
 *   m_l  = dense attention mass of each level-l node: sum over its tokens of
 *          softmax_t(q.k_t / sqrt(d)) over all n_tokens keys,
 *   pi_l = softmax over all level-l nodes of the router score max_j(q.s_j/sqrt(d) + c_j).
 * Readings (the pages give neither): KL(dense || router), over every node of a level; the
 * gradient of a node's score goes through its arg-max plane (lowest index on a tie); plain
 * SGD.  Work size: n_tokens * (Q + (levels + 1) * R) * d multiply-adds per KV head.
 *
 * zha_fit_workspace_bytes: bytes of the device fit workspace for this config, n_tokens and
 * nq (0 if invalid, or if nq * (Hq/Hkv) > 4096).  Host only.
 *
 * zha_fit_step:
 *   k_cache, v_cache  (device) [Hkv][capacity][d] dtype, as for zha_tree_build.
 *   n_tokens          1..capacity tokens the fit sees.
 *   ref_queries       (device) float32 [Hkv][R][d]: the master copy.  The tree is built from
 *                     its rounding to `dtype` (kept in fit_ws, which the handle then borrows
 *                     like zha_tree_build's reference queries); loss and gradient are taken
 *                     there; then ref_queries -= lr * grad in float32 (lr = 0: unchanged).
 *   q                 (device) [nq][Hq][d] dtype: training queries, query head h of the
 *                     group of KV head h / (Hq/Hkv).
 *   loss              (device) float32 [Hkv]: loss_kv at the rounded reference queries.
 *   grad              (device, nullable) float32 [Hkv][R][d]: its gradient.
 *   fit_ws            (device) >= zha_fit_workspace_bytes, 256-byte aligned; caller-owned.
 * The router fitted is the float32-plane one (with bf16 or FP4 router copies configured,
 * the build still writes them, and decode reads them).  Afterwards the handle holds a tree
 * over the rounded pre-update reference queries; rebuild with zha_tree_build to route with
 * the updated ones.  Errors as for zha_tree_build, plus ZHA_E_WORKSPACE for a short fit
 * workspace. */
size_t zha_fit_workspace_bytes(const zha_config* cfg, int64_t n_tokens, int64_t nq);
zha_status zha_fit_step(zha_tree* t, void* k_cache, void* v_cache, int64_t n_tokens, float* ref_queries,
                        const void* q, int64_t nq, float lr, float* loss, float* grad, void* fit_ws,
                        size_t fit_ws_bytes, hipStream_t stream);

/* One decode step for all query heads (blog, "Routing through the tree").
 *   q      (device) [Hq][d] dtype.
 *   out    (device) [Hq][d] float32: softmax attention over the routed tokens.
 *   stats  (device, nullable) int32 [levels + 1][Hkv]: row i < levels holds the size of
 *          the union (over the group's query heads) of the frontier scored at level
 *          levels - i; the last row holds the number of kept level-1 blocks (union).
 *          On the keys route (zha_route_mode 2) every node of every level is scored, so
 *          rows i < levels hold the level sizes.
 * Routing state stays on the device; nothing is read back to the host. */
zha_status zha_decode(zha_tree* t, const void* q, float* out, int32_t* stats,
                      hipStream_t stream);

/* Causal multi-query decode over a chunk of m new tokens (prefill with ZHA routing: the
 * method's attention cost is subquadratic in the context as a whole, blog, "How is this
 * subquadratic", and the paper's abstract).  For i = 0..m-1: appends token i
 * (k_new/v_new (device) [Hkv][m][d]
 * dtype, row i of each head) and decodes query row i (q (device) [m][Hq][d] dtype) into
 * out (device) [m][Hq][d] float32, so query i routes over the tree of the tokens up to
 * and including its own, exactly as m calls of zha_tree_append + zha_decode.
 * stats (nullable) [m][levels + 1][Hkv] as in zha_decode.  ZHA_E_CAPACITY when
 * N + m > capacity (nothing is enqueued).  All work is enqueued on `stream`; a HIP error
 * part-way leaves the tokens appended before it in the tree. */
zha_status zha_prefill(zha_tree* t, const void* k_new, const void* v_new, const void* q, float* out,
                       int64_t m, int32_t* stats, hipStream_t stream);

/* Bytes of device workspace zha_prefill_batched needs for sub-batches of up to `batch`
 * queries (1..128) over a tree of this config's capacity; 0 for an invalid config or
 * batch.  Dominated by the scores of every node for each (query, head) pair of a
 * sub-batch: about batch * Hq * (capacity / block) * 4 * b / (b - 1) bytes. */
size_t zha_prefill_workspace_bytes(const zha_config* cfg, int32_t batch);

/* Causal multi-query prefill, batched: the same result as zha_prefill (query i routes over
 * the tree of the tokens up to and including its own, blog, "Routing through the tree";
 * the routing of a whole prompt stays subquadratic, blog, "How is this subquadratic"),
 * computed `batch` queries at a time.  Per sub-batch of mb queries at positions
 * N0 .. N0+mb-1: the mb tokens are appended (cache rows and the nodes that cover them),
 * each query's own rightmost node of every level is built over the tokens up to its
 * position (the tree's node arithmetic: logsumexp of the children's log masses, their
 * softmax-weighted mean plane and offset), every node of every level is scored for all
 * mb * Hq (query, head) pairs in one pass over the planes, the nodes right of a pair's own
 * node drop out, each pair selects top-down with the fixed-point top-p rule of zha_decode,
 * and the routed attention of the mb queries runs in one launch, query i attending tokens
 * [0, N0 + i].  Scores use the float32 planes (whatever cfg.plane_dtype selects for decode).
 *   k_new, v_new  (device) [Hkv][m][d] dtype;  q (device) [m][Hq][d] dtype, 16-byte aligned;
 *   out           (device) [m][Hq][d] float32;
 *   batch         queries per sub-batch, 1..128;
 *   workspace     (device) at least zha_prefill_workspace_bytes(cfg, batch) bytes, 256-byte
 *                 aligned, owned by the caller; it holds the last sub-batch's scores and kept
 *                 bitmaps for zha_debug_prefill_trace until the next call that uses it.
 * ZHA_E_CAPACITY when N + m > capacity, ZHA_E_WORKSPACE when the workspace is too small
 * (nothing is enqueued).  All work is enqueued on `stream`; a HIP error part-way leaves
 * the sub-batches appended before it in the tree. */
zha_status zha_prefill_batched(zha_tree* t, const void* k_new, const void* v_new, const void* q, float* out,
                               int64_t m, int32_t batch, void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* The last sub-batch of zha_prefill_batched at `level` (1..levels), with mb its query
 * count, N its end (tokens in the tree after it) and P = mb * Hq / Hkv its pairs, in pair
 * order p = i * (Hq / Hkv) + head-in-group:
 *   scores  (device, nullable) float32 [Hkv][P][n], n = ceil(N / block^level): the router
 *           score of every node for every pair, -inf right of the pair's own node;
 *   kept    (device, nullable) uint32 [Hkv][P][ceil(n / 32)]: the pair's kept bitmap (bit
 *           e % 32 of word e / 32 = node e);
 *   own     (device, nullable) float32 [Hkv][mb][R][d + 2]: query i's own rightmost node of
 *           the level over the tokens up to its position, per plane (s [d], c, LSE).
 * ZHA_E_STATE when no batched prefill ran on this tree.  Reads the caller's prefill
 * workspace, which must still hold that call's contents. */
zha_status zha_debug_prefill_trace(zha_tree* t, int32_t level, float* scores, uint32_t* kept, float* own,
                                   hipStream_t stream);

/* Dense decode over all N tokens (the baseline attention the method is compared with):
 * out[h] = softmax(q_h.K^T/sqrt(d)) V for every query head. */
zha_status zha_decode_dense(zha_tree* t, const void* q, float* out, hipStream_t stream);

/* Dense decode as zha_decode_dense, allocation-free and without a handle or workspace: for
 * callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  The caller passes only inputs and outputs:
 *   cfg      (host) a valid config; head_dim, num_kv_heads, num_q_heads, capacity (the
 *            caches' row count) and dtype are used.
 *   k_cache, v_cache  (device) [Hkv][capacity][d] dtype; rows [0, n_tokens) are attended.
 *   q        (device) [Hq][d] dtype;  out (device) [Hq][d] float32.
 * Its split-K partials live in a fixed 4 MiB device array inside the library, one copy per
 * GPU, held until the process ends; the splits per KV head are capped so that
 * Hq * splits * (d + 2) * 4 bytes fit it.  ZHA_E_WORKSPACE if one split's partials
 * (Hq * (d + 2) * 4 bytes) exceed it.  No allocation, no synchronisation.  Calls that
 * overlap on one GPU (e.g. on two streams) share the array and race: serialise them. */
zha_status zha_decode_dense_static(const zha_config* cfg, const void* k_cache, const void* v_cache,
                                   int64_t n_tokens, const void* q, float* out, hipStream_t stream);

/* Sets the top-p threshold of each level for the following decodes (blog, "The narrow
 * path": a fixed fraction kept at every level compounds over the depth, so the threshold
 * has to change with depth and context; the pages give no formula, so the caller supplies
 * it).  p_levels (host) [levels]: entry l-1 is p at level l, each in (0, 1]; the values are
 * copied.  Null restores cfg.top_p at every level.  May be called at any time (before or
 * after build, between decodes); a context-dependent schedule p_l(N) is set before each
 * decode.  Host only; nothing is enqueued.  On error the schedule is left unchanged. */
zha_status zha_set_top_p_levels(zha_tree* t, const float* p_levels);

/* Chooses how the following decodes score the tree: mode 0 = the config's default
 * (zha_route_keys), 1 = per-level union frontiers (router planes, a level 1 from the keys
 * where zha_level1_key_form says so), 2 = every level from the keys.  Both modes compute
 * the same scores up to float32 rounding and apply the same selection rule.
 * ZHA_E_UNSUPPORTED for mode 2 on a config that cannot take it; ZHA_E_INVALID for another
 * mode.  Host only; nothing is enqueued; also used by zha_debug_route_level. */
zha_status zha_set_route_mode(zha_tree* t, int32_t mode);

/* The scoring the next decode uses: 1 = union frontiers, 2 = every level from the keys;
 * -1 for a null handle.  Host only. */
int32_t zha_route_mode(const zha_tree* t);

/* Copies level `level` (1..levels) of the tree into caller buffers:
 *   s_out (device) float32 [Hkv][n_l][R][d], c_out (device) float32 [Hkv][n_l][R] with
 *   n_l = ceil(N / block^level).  Enqueued copies only (no synchronisation). */
zha_status zha_debug_level(zha_tree* t, int32_t level, float* s_out, float* c_out,
                           hipStream_t stream);

/* Copies the quantised copy of s that routing reads at level `level`:
 *   ZHA_BF16:  s_out (device) bfloat16 [Hkv][n_l][R][d]; scale_out unused (may be null);
 *   ZHA_MXFP4: s_out (device) uint8 [Hkv][n_l][R][d/2], element 2i in the low 4 bits of
 *              byte i and element 2i+1 in the high 4 bits (E2M1 codes: bit 3 the sign,
 *              bits 0-2 the magnitude index into {0,.5,1,1.5,2,3,4,6});
 *              scale_out (device) uint8 [Hkv][n_l][R][d/32], the E8M0 block scales
 *              (X = 2^(byte - 127)).
 * ZHA_E_INVALID if the handle keeps no such copy at that level (float32 router planes, or
 * a level 1 scored from the keys).  Enqueued copies only (no synchronisation). */
zha_status zha_debug_router_planes(zha_tree* t, int32_t level, void* s_out, void* scale_out,
                                   hipStream_t stream);

/* Routing trace of the last zha_decode / zha_debug_route_level on this handle, for level
 * `level` (levels..1; 0 = the kept level-1 blocks).  Copies into caller device buffers
 * sized for `cap` entries per KV head:
 *   nodes  int32  [Hkv][cap]  node ids of the union frontier, ascending
 *   masks  uint32 [Hkv][cap]  bit i set: query head (kv*group + i) has the node in its
 *                             frontier (level 0: the head kept the block)
 *   scores float32[Hkv][8][cap] router score of each node for each query head of the
 *                             group (nullable; unused for level 0)
 *   keep   uint32 [Hkv][cap]  bit i set: query head i of the group kept the node
 *                             (nullable; unused for level 0)
 *   counts int32  [Hkv]       entries per KV head
 * ZHA_E_INVALID if cap is smaller than the level's node count. Synchronises `stream`. */
zha_status zha_debug_trace(zha_tree* t, int32_t level, int64_t cap, int32_t* nodes,
                           uint32_t* masks, float* scores, uint32_t* keep, int32_t* counts,
                           hipStream_t stream);

/* Teacher-forced routing of one level: scores the caller's union frontier (nodes/masks/
 * counts in the zha_debug_trace layout, with cap entries per KV head, device; node ids
 * ascending) for the queries q and applies the per-head top-p (blog, "Routing through the
 * tree"); results are read with zha_debug_trace at the same level.
 *   path 0: the kernels zha_decode runs at this level.  On the top levels it selects
 *           top-down (every level with at most 33,792 nodes up to the root, except a
 *           level 1 scored from the keys) every node of the level is scored and the trace
 *           holds every node (masks = the given frontier); elsewhere as path 1.
 *   path 1: the large-level kernels: the union list is scored, then the per-head
 *           histogram, boundary, classification and resolution launches.
 * Synchronises `stream`. */
zha_status zha_debug_route_level(zha_tree* t, int32_t level, const void* q,
                                 const int32_t* nodes, const uint32_t* masks,
                                 const int32_t* counts, int64_t cap, int32_t path,
                                 hipStream_t stream);

/* Launch timing for measurement.  zha_profile_start makes every later launch of this
 * handle whose key starts with `key_prefix` get a pair of HIP events on the launch's
 * stream.  Keys: "build_tile", "build_parent.l<level>", "append", "route_prep",
 * "route_score.l<level>", "route_select.l<level>" (histogram, boundary, classification
 * and resolution), "route_expand.l<level>", "attend" (split-K attention and combine),
 * "dense_attend".  zha_profile_stop synchronises on the recorded events and returns the
 * summed elapsed milliseconds and the number of bracketed launches (either pointer
 * nullable).  ZHA_E_STATE on start while active or stop while inactive. */
zha_status zha_profile_start(zha_tree* t, const char* key_prefix);
zha_status zha_profile_stop(zha_tree* t, double* total_ms, int64_t* launches);

/* Device invariant checks.  A library built with -DZHA_DEBUG (libzha_debug.so) compiles
 * checks into the same kernels: a list longer than its level's capacity, a list node outside
 * its level, a candidate or expanded list past its capacity, an attended block past N,
 * attention splits past their maximum, a top-down level past its size limit.  A failed check
 * sets its bit (bits 0..6 in that order) in the handle's check word; nothing traps.
 * zha_debug_check copies the word into *flags (host) and clears it; synchronises `stream`.
 * The word starts clear at each zha_tree_build in debug builds; in other builds it stays 0.
 * zha_debug_checks_compiled returns 1 in a debug build, else 0. */
zha_status zha_debug_check(zha_tree* t, uint32_t* flags, hipStream_t stream);
int32_t zha_debug_checks_compiled(void);

/* Tokens currently in the tree (host-side count; no synchronisation). */
int64_t zha_num_tokens(const zha_tree* t);

zha_status zha_destroy(zha_tree* t);
const char* zha_status_string(zha_status s);
const char* zha_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* ZHA_H */
