// Host side of the ZHA C ABI: argument validation, workspace layout, launch sequencing.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "../../include/zha.h"
#include "common.hpp"
#include "kernels.hpp"

using namespace zha;

// Event pairs around the launches whose key starts with the active prefix.
struct Profiler {
  bool on = false;
  std::string prefix;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> ev;
};

struct zha_tree {
  zha_config cfg;
  Profiler prof;
  char* ws;
  size_t ws_bytes;
  Dev dev;
  int64_t N;
  bool built;
  void* K;
  void* V;
  const void* refs;
  float top_p[MAXL + 1];  // p per level (index = level); cfg.top_p unless a schedule is set
  // the top-down selection of the last routing call: its route arguments, whether its
  // levels' dense union lists exist (they are written when a trace asks for them)
  RouteArgs td_args;
  bool td_valid;
  bool td_lists;
  // how decode scores the tree: 0 = by the config (allkeys_auto), 1 = frontier lists (planes,
  // key-form level 1), 2 = every level from the keys
  int32_t route_mode;
  // the last sub-batch of zha_prefill_batched (its buffers are in the caller's workspace)
  PrefillArgs pf_args;
  bool pf_valid;
};

namespace {

thread_local std::string g_err;

zha_status fail(zha_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

zha_status hip_fail(hipError_t e, const char* what) {
  return fail(ZHA_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int64_t MAX_CAPACITY = (int64_t)1 << 31;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// b^l, saturating at 2^62.
int64_t ipow_sat(int64_t b, int l) {
  int64_t r = 1;
  for (int i = 0; i < l; ++i) {
    if (r > ((int64_t)1 << 62) / b) return (int64_t)1 << 62;
    r *= b;
  }
  return r;
}

int64_t nodes_at(const zha_config& c, int level, int64_t n) { return ceil_div(n, ipow_sat(c.block, level)); }

// Level 1 is scored from the block's keys and the planes' token weights (q.s_j is the
// weighted sum of the block's logits q.k_t) when that reads fewer bytes than the planes:
// b keys plus R*b weights against R planes of d floats.  bf16 keys, b in {2, 4, 8, 16}.
bool key_form(const zha_config& c) {
  if (c.dtype != ZHA_BF16) return false;
  if (c.block != 2 && c.block != 4 && c.block != 8 && c.block != 16) return false;
  const int64_t keys = (int64_t)c.block * c.head_dim * 2 + (int64_t)c.num_ref * c.block * 4;
  const int64_t planes = (int64_t)c.num_ref * c.head_dim * 4;
  return keys < planes;
}

// Every level scored from the keys (allkeys.hip) is possible for block-4 key-form trees of at
// least AK_LC levels whose level 1 and levels above level 4 fit the top-down kernel's LDS.
bool allkeys_possible(const zha_config& c) {
  if (!key_form(c) || c.block != AK_B || c.levels < AK_LC) return false;
  if (c.num_ref % 4 || c.num_ref > 16) return false;
  if (nodes_at(c, 1, c.capacity) > AK_N1) return false;
  for (int l = 2; l <= c.levels; ++l)
    if (nodes_at(c, l, c.capacity) > TD_MAX) return false;
  int64_t dup = 0;
  for (int l = AK_LC + 1; l <= c.levels; ++l) dup += nodes_at(c, l, c.capacity) * c.num_ref;
  return dup <= AK_DUP;
}

// Bytes one decode reads to score every level from the keys, against the other path with
// its level-1 frontier covering the whole level (its upper levels are scored whole anyway):
// keys and token weights per token, (c, LSE) per node of levels 1..4, against the router
// planes of levels 2..L plus the level-1 keys, token weights and offsets.  Counted at
// capacity.
bool allkeys_auto(const zha_config& c) {
  if (!allkeys_possible(c)) return false;
  const int64_t R = c.num_ref, D = c.head_dim, n = c.capacity;
  int64_t keys = n * (2 * D + 4 * R);
  for (int l = 1; l <= AK_LC; ++l) keys += nodes_at(c, l, n) * 8 * R;
  const int64_t plane = c.plane_dtype == ZHA_BF16 ? R * (2 * D + 4)
                        : c.plane_dtype == ZHA_MXFP4 ? R * (D / 2 + D / 32 + 4)
                                                     : R * (D + 1) * 4;
  int64_t other = n * (2 * D + 4 * R) + nodes_at(c, 1, n) * 4 * R;
  for (int l = 2; l <= c.levels; ++l) other += nodes_at(c, l, n) * plane;
  return keys <= other;
}

int tile_tokens(const zha_config& c) { return c.block <= 128 ? 128 : 256; }

int tile_levels(const zha_config& c) {
  const int T = tile_tokens(c);
  int m = 0;
  int64_t span = 1;
  while (m < c.levels && span * c.block <= T) { span *= c.block; ++m; }
  return m;
}

zha_status validate(const zha_config* c) {
  if (!c) return fail(ZHA_E_INVALID, "config is null");
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(ZHA_E_UNSUPPORTED, "head_dim %d not built (64 or 128)", c->head_dim);
  if (c->num_kv_heads < 1) return fail(ZHA_E_INVALID, "num_kv_heads %d < 1", c->num_kv_heads);
  if (c->num_q_heads < c->num_kv_heads || c->num_q_heads % c->num_kv_heads)
    return fail(ZHA_E_INVALID, "num_q_heads %d is not a multiple of num_kv_heads %d", c->num_q_heads,
                c->num_kv_heads);
  if (c->num_q_heads / c->num_kv_heads > GMAX)
    return fail(ZHA_E_UNSUPPORTED, "group size %d > %d", c->num_q_heads / c->num_kv_heads, GMAX);
  if (c->block < 2 || c->block > 256) return fail(ZHA_E_INVALID, "block %d outside 2..256", c->block);
  // the build summarises 128- or 256-token tiles whose nodes must start on tile boundaries
  if (c->block & (c->block - 1))
    return fail(ZHA_E_UNSUPPORTED, "block %d is not a power of two", c->block);
  if (c->levels < 1 || c->levels > MAXL) return fail(ZHA_E_INVALID, "levels %d outside 1..%d", c->levels, MAXL);
  if (c->num_ref != 1 && c->num_ref != 2 && c->num_ref != 4 && c->num_ref != 8 && c->num_ref != 16)
    return fail(ZHA_E_UNSUPPORTED, "num_ref %d not built (1, 2, 4, 8, 16)", c->num_ref);
  if (c->capacity < 1 || c->capacity >= MAX_CAPACITY)
    return fail(ZHA_E_INVALID, "capacity %lld outside 1..2^31-1", (long long)c->capacity);
  if (c->dtype != ZHA_F32 && c->dtype != ZHA_BF16) return fail(ZHA_E_INVALID, "dtype %d", c->dtype);
  if (!(c->top_p > 0.f && c->top_p <= 1.f)) return fail(ZHA_E_INVALID, "top_p %g outside (0, 1]", c->top_p);
  if (c->keep_sink != 0 && c->keep_sink != 1) return fail(ZHA_E_INVALID, "keep_sink %d", c->keep_sink);
  if (c->plane_dtype != ZHA_F32 && c->plane_dtype != ZHA_BF16 && c->plane_dtype != ZHA_MXFP4)
    return fail(ZHA_E_INVALID, "plane_dtype %d", c->plane_dtype);
  if (c->dtype == ZHA_F32 && c->head_dim == 128 && c->block > 128)
    return fail(ZHA_E_UNSUPPORTED, "float32 keys with head_dim 128 need block <= 128");
  return ZHA_OK;
}

// Lays the workspace out; with base == nullptr only the size is computed.
size_t layout(const zha_config& c, char* base, Dev* dev) {
  size_t off = 0;
  auto take = [&](size_t bytes) -> char* {
    off = (off + 255) & ~(size_t)255;
    char* p = base ? base + off : nullptr;
    off += bytes;
    return p;
  };
  Dev d;
  memset(&d, 0, sizeof d);
  const int64_t H = c.num_kv_heads, Q = c.num_q_heads, R = c.num_ref, D = c.head_dim;
  const int L = c.levels;
  // per-level strides rounded to 64 nodes: every per-head row starts 256-byte aligned
  for (int l = 1; l <= L; ++l) d.ncap[l] = ceil_div(nodes_at(c, l, c.capacity), 64) * 64;
  d.ncap[0] = d.ncap[1];
  for (int l = 1; l <= L; ++l) {
    d.s[l] = (float*)take((size_t)(H * d.ncap[l] * R * D) * 4);
    d.c[l] = (float*)take((size_t)(H * d.ncap[l] * R) * 4);
    d.lse[l] = (float*)take((size_t)(H * d.ncap[l] * R) * 4);
  }
  for (int l = 0; l <= L; ++l) {
    d.node[l] = (int32_t*)take((size_t)(H * d.ncap[l]) * 4);
    d.mask[l] = (uint32_t*)take((size_t)(H * d.ncap[l]) * 4);
    if (l >= 1) {
      d.keep[l] = (uint32_t*)take((size_t)(H * d.ncap[l]) * 4);
      d.score[l] = (float*)take((size_t)(H * GMAX * d.ncap[l]) * 4);
      d.part[l] = (int32_t*)take((size_t)(H * ceil_div(d.ncap[l], EXPAND_CHUNK)) * 4);
    }
  }
  if (key_form(c)) d.w1 = (float*)take((size_t)(H * d.ncap[1] * R * c.block) * 4);
  if (c.plane_dtype == ZHA_BF16)
    for (int l = key_form(c) ? 2 : 1; l <= L; ++l) d.sq[l] = (bf16_t*)take((size_t)(H * d.ncap[l] * R * D) * 2);
  if (c.plane_dtype == ZHA_MXFP4)
    for (int l = key_form(c) ? 2 : 1; l <= L; ++l) {
      d.s4[l] = (uint8_t*)take((size_t)(H * d.ncap[l] * R * D) / 2);
      d.s4x[l] = (uint8_t*)take((size_t)(H * d.ncap[l] * R * D) / 32);
    }
  d.cnt = (int32_t*)take((size_t)((MAXL + 1) * H) * 4);
  d.ucnt = (int32_t*)take((size_t)((MAXL + 1) * H) * 4);
  d.qs = (QState*)take((size_t)((L + 1) * Q) * sizeof(QState));
  d.hpart = (uint64_t*)take((size_t)(H * SEL_P * GMAX * NB1) * 8);
  d.tdbits = (uint32_t*)take((size_t)((L + 1) * Q * 2 * TD_WORDS) * 4);
  if (allkeys_possible(c)) {
    d.kb1 = (uint32_t*)take((size_t)(Q * 2 * (d.ncap[1] / 32)) * 4);
    d.kdots = (float*)take((size_t)(H * d.ncap[AK_LC] * GMAX * R) * 4);
    d.tick = (uint32_t*)take((size_t)H * 4);
  }
  d.sib = (float*)take((size_t)(H * SIB_STRIDE(R, D)) * 4);
  d.sibkey = (int64_t*)take((size_t)(H * (MAXL + 1)) * 8);
  d.cand = (int32_t*)take((size_t)(Q * d.ncap[1]) * 4);
  d.qf = (float*)take((size_t)(Q * D) * 4);
  d.apart = (float*)take((size_t)(Q * MAX_SPLITS * (D + 2)) * 4);
  d.err = (uint32_t*)take(256);
  if (dev) *dev = d;
  return (off + 255) & ~(size_t)255;
}

int attn_splits(int64_t tokens, int64_t per_split, int max_splits) {
  int64_t s = ceil_div(tokens, per_split);
  if (s < 1) s = 1;
  if (s > max_splits) s = max_splits;
  return (int)s;
}

RouteArgs route_args(const zha_tree* t, const void* q) {
  RouteArgs a;
  memset(&a, 0, sizeof a);
  a.dev = t->dev;
  a.q = q;
  a.N = t->N;
  a.hkv = t->cfg.num_kv_heads;
  a.hq = t->cfg.num_q_heads;
  a.g = a.hq / a.hkv;
  a.b = t->cfg.block;
  a.levels = t->cfg.levels;
  for (int l = 0; l <= MAXL; ++l) a.top_p[l] = t->top_p[l];
  a.sigma = 1.0f / sqrtf((float)t->cfg.head_dim);
  a.key_form = key_form(t->cfg) ? 1 : 0;
  a.nref = t->cfg.num_ref;
  a.allkeys = t->route_mode == 2 || (t->route_mode == 0 && allkeys_auto(t->cfg)) ? 1 : 0;
  a.q_bf16 = t->cfg.dtype == ZHA_BF16 ? 1 : 0;
  a.planes = t->cfg.plane_dtype;
  a.K = t->K;
  a.kcap = t->cfg.capacity;
  for (int l = 1; l <= t->cfg.levels; ++l) a.nl[l] = nodes_at(t->cfg, l, t->N);
  a.nl[0] = a.nl[1];
  return a;
}

// Brackets one launch with events when profiling covers `key`.
struct ProfScope {
  zha_tree* t;
  hipStream_t st;
  hipEvent_t a = nullptr, b = nullptr;
  ProfScope(zha_tree* t_, const std::string& key, hipStream_t s) : t(t_), st(s) {
    if (!t->prof.on || key.compare(0, t->prof.prefix.size(), t->prof.prefix) != 0) return;
    if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) { a = b = nullptr; return; }
    (void)hipEventRecord(a, st);
  }
  ~ProfScope() {
    if (!a) return;
    (void)hipEventRecord(b, st);
    t->prof.ev.emplace_back(a, b);
  }
};

// Lowest level of the top levels that zha_decode scores whole and selects top-down: every
// level from there up has at most TD_MAX nodes (a key-form level 1 keeps its own kernel).
int topdown_lo(const RouteArgs& r) {
  int lo = r.levels + 1;
  while (lo > 1 && r.nl[lo - 1] <= TD_MAX) --lo;
  if (r.key_form && lo == 1) lo = 2;
  return lo;
}

std::string lvkey(const char* name, int lv) { return std::string(name) + ".l" + std::to_string(lv); }

zha_status route_levels(zha_tree* t, RouteArgs& a, int lv, hipStream_t st, bool expand) {
  a.level = lv;
  a.nlevel = nodes_at(t->cfg, lv, t->N);
  a.nbelow = lv > 1 ? nodes_at(t->cfg, lv - 1, t->N) : 0;
  hipError_t e;
  {
    ProfScope ps(t, lvkey("route_score", lv), st);
    e = launch_route_score(a, t->cfg.head_dim, t->cfg.num_ref, st);
  }
  if (e != hipSuccess) return hip_fail(e, "route score launch");
  {
    ProfScope ps(t, lvkey("route_select", lv), st);
    e = launch_route_select(a, st);
  }
  if (e != hipSuccess) return hip_fail(e, "route select launch");
  if (expand) {
    ProfScope ps(t, lvkey("route_expand", lv), st);
    e = launch_route_expand(a, st);
  }
  if (e != hipSuccess) return hip_fail(e, "route expand launch");
  return ZHA_OK;
}

}  // namespace

extern "C" {

int32_t zha_level1_key_form(const zha_config* cfg) {
  if (validate(cfg) != ZHA_OK) return -1;
  return key_form(*cfg) ? 1 : 0;
}

int32_t zha_route_keys(const zha_config* cfg) {
  if (validate(cfg) != ZHA_OK) return -1;
  return allkeys_auto(*cfg) ? 1 : 0;
}

zha_status zha_set_route_mode(zha_tree* t, int32_t mode) {
  if (!t) return fail(ZHA_E_INVALID, "tree is null");
  if (mode < 0 || mode > 2) return fail(ZHA_E_INVALID, "route mode %d outside 0..2", mode);
  if (mode == 2 && !allkeys_possible(t->cfg))
    return fail(ZHA_E_UNSUPPORTED, "this config cannot score every level from the keys");
  t->route_mode = mode;
  t->td_valid = false;
  return ZHA_OK;
}

int32_t zha_route_mode(const zha_tree* t) {
  if (!t) return -1;
  return (t->route_mode == 2 || (t->route_mode == 0 && allkeys_auto(t->cfg))) ? 2 : 1;
}

size_t zha_workspace_bytes(const zha_config* cfg) {
  if (validate(cfg) != ZHA_OK) return 0;
  return layout(*cfg, nullptr, nullptr);
}

zha_status zha_create(const zha_config* cfg, void* workspace, size_t workspace_bytes, zha_tree** out) {
  zha_status s = validate(cfg);
  if (s != ZHA_OK) return s;
  if (!out) return fail(ZHA_E_INVALID, "out is null");
  if (!workspace) return fail(ZHA_E_INVALID, "workspace is null");
  if ((uintptr_t)workspace % 256) return fail(ZHA_E_INVALID, "workspace not 256-byte aligned");
  const size_t need = layout(*cfg, nullptr, nullptr);
  if (workspace_bytes < need)
    return fail(ZHA_E_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  zha_tree* t = new (std::nothrow) zha_tree();
  if (!t) return fail(ZHA_E_INVALID, "host allocation failed");
  t->cfg = *cfg;
  for (int l = 0; l <= MAXL; ++l) t->top_p[l] = cfg->top_p;
  t->ws = (char*)workspace;
  t->ws_bytes = workspace_bytes;
  layout(*cfg, t->ws, &t->dev);
  *out = t;
  return ZHA_OK;
}

}  // extern "C"

namespace {

// Builds every node that covers a token in [from, to) (from = 0: the whole tree over
// [0, to)): the key tiles from the one holding token `from`, the parents from the one
// holding it, and the FP4 router copies of those nodes.
zha_status enqueue_build(zha_tree* t, const void* k_cache, const void* refs, int64_t from, int64_t to,
                         hipStream_t stream) {
  const zha_config& c = t->cfg;
  BuildArgs a;
  memset(&a, 0, sizeof a);
  a.K = k_cache;
  a.refs = refs;
  a.cap = c.capacity;
  a.N = to;
  a.b = c.block;
  a.sigma = 1.0f / sqrtf((float)c.head_dim);
  a.dev = t->dev;
  const bool narrow = narrow_build(c.num_ref, c.block);
  a.m = narrow ? (c.levels < 2 ? c.levels : 2) : tile_levels(c);
  const int T = narrow ? narrow_tile_tokens(c.head_dim, c.block) : tile_tokens(c);
  a.tile0 = from / T;
  hipError_t e;
  {
    ProfScope ps(t, "build_tile", stream);
    e = narrow ? launch_build_narrow(a, c.dtype == ZHA_BF16, c.head_dim, c.num_ref, c.num_kv_heads, stream)
               : launch_build_tile(a, c.dtype == ZHA_BF16, c.head_dim, c.num_ref, ceil_div(to, T), c.num_kv_heads, T,
                                   stream);
  }
  if (e != hipSuccess) return hip_fail(e, "build tile launch");
  for (int v = a.m + 1; v <= c.levels; ++v) {
    ParentArgs p;
    memset(&p, 0, sizeof p);
    p.dev = t->dev;
    p.level = v;
    p.b = c.block;
    p.nparent = nodes_at(c, v, to);
    p.nchild = nodes_at(c, v - 1, to);
    p.first = from / ipow_sat(c.block, v);
    {
      ProfScope ps(t, lvkey("build_parent", v), stream);
      e = launch_build_parent(p, c.head_dim, c.num_ref, c.num_kv_heads, stream);
    }
    if (e != hipSuccess) return hip_fail(e, "build parent launch");
  }
  // FP4 router copies of the rebuilt nodes of every routed level, from the finished planes
  // (the narrow leaf kernel writes those of its own levels itself)
  for (int v = narrow ? a.m + 1 : 1; v <= c.levels; ++v) {
    if (!t->dev.s4[v]) continue;
    QuantArgs q;
    memset(&q, 0, sizeof q);
    q.dev = t->dev;
    q.level = v;
    q.first = from / ipow_sat(c.block, v);
    q.nnode = nodes_at(c, v, to);
    {
      ProfScope ps(t, lvkey("build_quant", v), stream);
      e = launch_quantise_fp4(q, c.head_dim, c.num_ref, c.num_kv_heads, stream);
    }
    if (e != hipSuccess) return hip_fail(e, "fp4 quantise launch");
  }
  return ZHA_OK;
}

constexpr int64_t FIT_MAX_Q = 4096;   // training queries per KV head in one fitting step

// Lays out the fit workspace for n_tokens tokens and nq training queries per head; with
// base == nullptr only the size is computed.
size_t fit_layout(const zha_config& c, int64_t N, int64_t nq, char* base, FitArgs* fa) {
  size_t off = 0;
  auto take = [&](size_t bytes) -> char* {
    off = (off + 255) & ~(size_t)255;
    char* p = base ? base + off : nullptr;
    off += bytes;
    return p;
  };
  FitArgs a;
  memset(&a, 0, sizeof a);
  const int64_t H = c.num_kv_heads, R = c.num_ref, D = c.head_dim, g = c.num_q_heads / c.num_kv_heads;
  const int64_t Q = nq * g;
  const int L = c.levels;
  a.refs_in = take((size_t)(H * R * D) * 4);
  a.refs_r = (float*)take((size_t)(H * R * D) * 4);
  a.qf = (float*)take((size_t)(H * Q * D) * 4);
  a.zstride = ceil_div(N, 64) * 64;
  a.z = (float*)take((size_t)(H * Q * a.zstride) * 4);
  for (int l = 1; l <= L; ++l) {
    a.nl[l] = nodes_at(c, l, N);
    a.nstride[l] = ceil_div(a.nl[l], 64) * 64;
    a.lt[l] = (float*)take((size_t)(H * Q * a.nstride[l]) * 4);
    a.sc[l] = (float*)take((size_t)(H * Q * a.nstride[l]) * 4);
    a.gr[l] = (float*)take((size_t)(H * Q * a.nstride[l]) * 4);
    a.am[l] = (uint8_t*)take((size_t)(H * Q * a.nstride[l]));
    a.wb[l] = (float*)take((size_t)(H * a.nstride[l] * R * 2) * 4);
  }
  a.kl = (float*)take((size_t)(H * Q * L) * 4);
  a.alpha = (float*)take((size_t)(H * N * R) * 4);
  a.nchunk = (int32_t)ceil_div(N, fit_chunk_tokens());
  a.part = (float*)take((size_t)(H * a.nchunk * R * D) * 4);
  a.grad = (float*)take((size_t)(H * R * D) * 4);   // used when the caller wants no gradient
  a.N = N;
  a.Q = (int32_t)Q;
  if (fa) *fa = a;
  return (off + 255) & ~(size_t)255;
}

}  // namespace

extern "C" {

size_t zha_fit_workspace_bytes(const zha_config* cfg, int64_t n_tokens, int64_t nq) {
  if (validate(cfg) != ZHA_OK) return 0;
  if (n_tokens < 1 || n_tokens > cfg->capacity || nq < 1) return 0;
  if (nq * (cfg->num_q_heads / cfg->num_kv_heads) > FIT_MAX_Q) return 0;
  return fit_layout(*cfg, n_tokens, nq, nullptr, nullptr);
}

zha_status zha_fit_step(zha_tree* t, void* k_cache, void* v_cache, int64_t n_tokens, float* ref_queries,
                        const void* q, int64_t nq, float lr, float* loss, float* grad, void* fit_ws,
                        size_t fit_ws_bytes, hipStream_t stream) {
  if (!t) return fail(ZHA_E_INVALID, "tree is null");
  const zha_config& c = t->cfg;
  if (!k_cache || !v_cache || !ref_queries || !q || !loss || !fit_ws)
    return fail(ZHA_E_INVALID, "null cache, reference-query, query, loss or workspace pointer");
  if (((uintptr_t)k_cache | (uintptr_t)v_cache | (uintptr_t)ref_queries | (uintptr_t)q | (uintptr_t)grad) % 16)
    return fail(ZHA_E_INVALID, "cache, reference-query, query and gradient pointers must be 16-byte aligned");
  if ((uintptr_t)fit_ws % 256) return fail(ZHA_E_INVALID, "fit workspace not 256-byte aligned");
  if (n_tokens < 1) return fail(ZHA_E_INVALID, "n_tokens %lld < 1", (long long)n_tokens);
  if (n_tokens > c.capacity)
    return fail(ZHA_E_CAPACITY, "n_tokens %lld > capacity %lld", (long long)n_tokens, (long long)c.capacity);
  const int64_t g = c.num_q_heads / c.num_kv_heads;
  if (nq < 1 || nq * g > FIT_MAX_Q)
    return fail(ZHA_E_INVALID, "nq %lld: between 1 and %lld training queries per KV head", (long long)nq,
                (long long)(FIT_MAX_Q / g));
  if (!std::isfinite(lr)) return fail(ZHA_E_INVALID, "lr is not finite");
  const size_t need = fit_layout(c, n_tokens, nq, nullptr, nullptr);
  if (fit_ws_bytes < need)
    return fail(ZHA_E_WORKSPACE, "fit workspace %zu bytes < %zu needed", fit_ws_bytes, need);
  FitArgs a;
  fit_layout(c, n_tokens, nq, (char*)fit_ws, &a);
  a.K = k_cache;
  a.q = q;
  a.refs_master = ref_queries;
  a.loss = loss;
  if (grad) a.grad = grad;
  a.cap = c.capacity;
  a.hkv = c.num_kv_heads;
  a.hq = c.num_q_heads;
  a.g = (int32_t)g;
  a.b = c.block;
  a.levels = c.levels;
  a.R = c.num_ref;
  a.D = c.head_dim;
  a.sigma = 1.0f / sqrtf((float)c.head_dim);
  a.lr = lr;
  const bool bf16 = c.dtype == ZHA_BF16;
  hipError_t e;
  {
    ProfScope ps(t, "fit.cast", stream);
    e = launch_fit_cast_refs(a, bf16, stream);
  }
  if (e != hipSuccess) return hip_fail(e, "fit cast launch");
  zha_status zs = enqueue_build(t, k_cache, a.refs_in, 0, n_tokens, stream);
  if (zs != ZHA_OK) return zs;
  t->K = k_cache;
  t->V = v_cache;
  t->refs = a.refs_in;
  t->N = n_tokens;
  t->built = true;
  a.dev = t->dev;
  static const char* const stage_key[FIT_NSTAGE] = {"fit.logits", "fit.mass", "fit.score", "fit.loss", "fit.alpha",
                                                     "fit.grad"};
  for (int stage = 0; stage < FIT_NSTAGE; ++stage) {
    {
      ProfScope ps(t, stage_key[stage], stream);
      e = launch_fit_stage(a, bf16, stage, stream);
    }
    if (e != hipSuccess) return hip_fail(e, stage_key[stage]);
  }
  return ZHA_OK;
}

zha_status zha_tree_build(zha_tree* t, void* k_cache, void* v_cache, int64_t n_tokens, const void* ref_queries,
                          hipStream_t stream) {
  if (!t) return fail(ZHA_E_INVALID, "tree is null");
  if (!k_cache || !v_cache || !ref_queries) return fail(ZHA_E_INVALID, "null cache or reference-query pointer");
  if (((uintptr_t)k_cache | (uintptr_t)v_cache | (uintptr_t)ref_queries) % 16)
    return fail(ZHA_E_INVALID, "cache and reference-query pointers must be 16-byte aligned");
  if (n_tokens < 1) return fail(ZHA_E_INVALID, "n_tokens %lld < 1", (long long)n_tokens);
  if (n_tokens > t->cfg.capacity)
    return fail(ZHA_E_CAPACITY, "n_tokens %lld > capacity %lld", (long long)n_tokens, (long long)t->cfg.capacity);
#ifdef ZHA_DEBUG
  {
    hipError_t e = hipMemsetAsync(t->dev.err, 0, 4, stream);   // debug builds: checks start clear
    if (e != hipSuccess) return hip_fail(e, "check word");
  }
#endif
  zha_status zs = enqueue_build(t, k_cache, ref_queries, 0, n_tokens, stream);
  if (zs != ZHA_OK) return zs;
  t->K = k_cache;
  t->V = v_cache;
  t->refs = ref_queries;
  t->N = n_tokens;
  t->built = true;
  return ZHA_OK;
}

zha_status zha_tree_append_n(zha_tree* t, const void* k_new, const void* v_new, int64_t m, hipStream_t stream) {
  if (!t) return fail(ZHA_E_INVALID, "tree is null");
  if (!t->built) return fail(ZHA_E_STATE, "append before build");
  if (!k_new || !v_new) return fail(ZHA_E_INVALID, "null k_new or v_new");
  if (m < 1) return fail(ZHA_E_INVALID, "m %lld < 1", (long long)m);
  if (t->N + m > t->cfg.capacity)
    return fail(ZHA_E_CAPACITY, "%lld + %lld tokens > capacity %lld", (long long)t->N, (long long)m,
                (long long)t->cfg.capacity);
  const zha_config& c = t->cfg;
  const size_t es = c.dtype == ZHA_BF16 ? 2 : 4, row = (size_t)c.head_dim * es;
  // rows N .. N+m-1 of every KV head's caches
  hipError_t e = hipMemcpy2DAsync((char*)t->K + (size_t)t->N * row, (size_t)c.capacity * row, k_new, (size_t)m * row,
                                  (size_t)m * row, c.num_kv_heads, hipMemcpyDeviceToDevice, stream);
  if (e == hipSuccess)
    e = hipMemcpy2DAsync((char*)t->V + (size_t)t->N * row, (size_t)c.capacity * row, v_new, (size_t)m * row,
                         (size_t)m * row, c.num_kv_heads, hipMemcpyDeviceToDevice, stream);
  if (e != hipSuccess) return hip_fail(e, "cache row copy");
  zha_status zs = enqueue_build(t, t->K, t->refs, t->N, t->N + m, stream);
  if (zs != ZHA_OK) return zs;
  t->N += m;
  return ZHA_OK;
}

}  // extern "C"

namespace {

// One-token append (validated by the caller); the new row of KV head kv is at
// k_new + kv * stride elements.
zha_status enqueue_append(zha_tree* t, const void* k_new, const void* v_new, int64_t stride, hipStream_t stream) {
  const zha_config& c = t->cfg;
  AppendArgs a;
  memset(&a, 0, sizeof a);
  a.K = t->K;
  a.V = t->V;
  a.k_new = k_new;
  a.v_new = v_new;
  a.new_stride = stride;
  a.refs = t->refs;
  a.cap = c.capacity;
  a.N = t->N;
  a.b = c.block;
  a.levels = c.levels;
  a.sigma = 1.0f / sqrtf((float)c.head_dim);
  a.dev = t->dev;
  hipError_t e;
  {
    ProfScope ps(t, "append", stream);
    e = launch_append(a, c.dtype == ZHA_BF16, c.head_dim, c.num_ref, c.num_kv_heads, stream);
  }
  if (e != hipSuccess) return hip_fail(e, "append launch");
  t->N += 1;
  return ZHA_OK;
}

}  // namespace

extern "C" {

zha_status zha_tree_append(zha_tree* t, const void* k_new, const void* v_new, hipStream_t stream) {
  if (!t) return fail(ZHA_E_INVALID, "tree is null");
  if (!t->built) return fail(ZHA_E_STATE, "append before build");
  if (!k_new || !v_new) return fail(ZHA_E_INVALID, "null k_new or v_new");
  if (t->N >= t->cfg.capacity) return fail(ZHA_E_CAPACITY, "cache full (%lld tokens)", (long long)t->N);
  return enqueue_append(t, k_new, v_new, t->cfg.head_dim, stream);
}

zha_status zha_decode(zha_tree* t, const void* q, float* out, int32_t* stats, hipStream_t stream) {
  if (!t) return fail(ZHA_E_INVALID, "tree is null");
  if (!t->built) return fail(ZHA_E_STATE, "decode before build");
  if (!q || !out) return fail(ZHA_E_INVALID, "null q or out");
  if ((uintptr_t)q % 16) return fail(ZHA_E_INVALID, "q must be 16-byte aligned");
  const zha_config& c = t->cfg;
  RouteArgs r = route_args(t, q);
  r.nlevel = nodes_at(c, c.levels, t->N);
  // top levels small enough to score whole and select top-down in one launch (every level
  // when all are scored from the keys)
  const int lo = r.allkeys ? 1 : topdown_lo(r);
  r.dense_lo = lo <= c.levels ? lo : 0;   // prep sets the list sizes of those levels
  hipError_t e = hipSuccess;
  if (!r.allkeys) {
    ProfScope ps(t, "route_prep", stream);
    e = launch_route_prep(r, c.dtype == ZHA_BF16, c.head_dim, stream);
  }
  if (e != hipSuccess) return hip_fail(e, "route prep launch");
  t->td_valid = false;
  if (r.allkeys) {
    // (no prep launch: the score kernel's first workgroup sets the list sizes and clears the
    // selection's arrival counts; nothing else of the prep is read on this path)
    r.prep_fold = 1;
    // levels 1..4 and the level-4 dot products from one pass over the keys; the levels above
    // derived and every level selected top-down; the union of the kept blocks written by the
    // selection's last workgroup of each KV head
    r.level = c.levels;
    {
      ProfScope ps(t, "route_score.keys", stream);
      e = launch_route_allkeys_score(r, c.head_dim, c.num_ref, stream);
    }
    if (e != hipSuccess) return hip_fail(e, "route key score launch");
    {
      ProfScope ps(t, "route_select.keys", stream);
      e = launch_route_topdown_keys(r, stream);
    }
    if (e != hipSuccess) return hip_fail(e, "route top-down select launch");
    t->td_args = r;
    t->td_valid = true;
    t->td_lists = false;
  } else if (lo <= c.levels) {
    r.level = c.levels;
    r.dense = 1;
    {
      ProfScope ps(t, "route_score.top", stream);
      e = launch_route_dense_score(r, c.head_dim, c.num_ref, stream);
    }
    if (e != hipSuccess) return hip_fail(e, "route dense score launch");
    {
      ProfScope ps(t, "route_select.top", stream);
      e = launch_route_topdown(r, stream);
    }
    if (e != hipSuccess) return hip_fail(e, "route top-down select launch");
    r.dense = 0;
    t->td_args = r;
    t->td_valid = true;
    t->td_lists = false;
    if (lo >= 2) {
      // the next level's union list straight from the kept bitmaps
      ProfScope ps(t, "route_expand.top", stream);
      e = launch_route_td_children(r, stream);
    } else {
      // level 1 selected top-down: its dense lists, then the gather list
      ProfScope ps(t, "route_expand.top", stream);
      e = launch_route_td_lists(r, stream);
      t->td_lists = true;
      r.level = lo;
      r.nlevel = r.nl[lo];
      r.nbelow = 0;
      if (e == hipSuccess) e = launch_route_expand(r, stream);
    }
    if (e != hipSuccess) return hip_fail(e, "route top-down list launch");
  }
  for (int lv = lo - 1; lv >= 1; --lv) {
    zha_status s = route_levels(t, r, lv, stream, true);
    if (s != ZHA_OK) return s;
  }
  AttnArgs a;
  memset(&a, 0, sizeof a);
  a.dev = t->dev;
  a.K = t->K;
  a.V = t->V;
  a.q = q;
  a.cap = c.capacity;
  a.N = t->N;
  a.hkv = c.num_kv_heads;
  a.hq = c.num_q_heads;
  a.g = a.hq / a.hkv;
  a.b = c.block;
  // one wave of resident workgroups; splits beyond the gathered tokens exit at once
  a.splits = attend_resident_splits(c.dtype == ZHA_BF16, c.head_dim, false, c.num_kv_heads);
  a.keep_sink = c.keep_sink;
  a.pstride = MAX_SPLITS;
  a.sigma = 1.0f / sqrtf((float)c.head_dim);
  a.out = out;
  {
    ProfScope ps(t, "attend", stream);
    e = launch_attend_full(a, c.dtype == ZHA_BF16, c.head_dim, false, stats, c.levels, stream);
  }
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return ZHA_OK;
}

zha_status zha_prefill(zha_tree* t, const void* k_new, const void* v_new, const void* q, float* out, int64_t m,
                       int32_t* stats, hipStream_t stream) {
  if (!t) return fail(ZHA_E_INVALID, "tree is null");
  if (!t->built) return fail(ZHA_E_STATE, "prefill before build");
  if (!k_new || !v_new || !q || !out) return fail(ZHA_E_INVALID, "null k_new, v_new, q or out");
  if ((uintptr_t)q % 16) return fail(ZHA_E_INVALID, "q must be 16-byte aligned");
  if (m < 1) return fail(ZHA_E_INVALID, "m %lld < 1", (long long)m);
  if (t->N + m > t->cfg.capacity)
    return fail(ZHA_E_CAPACITY, "%lld + %lld tokens > capacity %lld", (long long)t->N, (long long)m,
                (long long)t->cfg.capacity);
  const zha_config& c = t->cfg;
  const size_t es = c.dtype == ZHA_BF16 ? 2 : 4, d = (size_t)c.head_dim;
  for (int64_t i = 0; i < m; ++i) {
    // token i: row i of each KV head's [m][d] chunk
    zha_status zs = enqueue_append(t, (const char*)k_new + (size_t)i * d * es, (const char*)v_new + (size_t)i * d * es,
                                   m * (int64_t)d, stream);
    if (zs != ZHA_OK) return zs;
    zs = zha_decode(t, (const char*)q + (size_t)i * c.num_q_heads * d * es, out + (size_t)i * c.num_q_heads * d,
                    stats ? stats + (size_t)i * (c.levels + 1) * c.num_kv_heads : nullptr, stream);
    if (zs != ZHA_OK) return zs;
  }
  return ZHA_OK;
}

}  // extern "C"

namespace {

constexpr int PF_MAX_BATCH = 128;   // queries per sub-batch
constexpr int PF_SPLITS = 16;       // attention splits per query and KV head, at most

// Lays out the batched-prefill workspace for sub-batches of up to `mbmax` queries; with
// base == nullptr only the size is computed.  Level strides follow the tree's node
// capacities, so every row starts 256-byte aligned.
size_t prefill_layout(const zha_config& c, int mbmax, char* base, PrefillArgs* out, float** apart, int* pstride,
                      float** upart = nullptr) {
  size_t off = 0;
  auto take = [&](size_t bytes) -> char* {
    off = (off + 255) & ~(size_t)255;
    char* p = base ? base + off : nullptr;
    off += bytes;
    return p;
  };
  PrefillArgs a;
  memset(&a, 0, sizeof a);
  const int64_t H = c.num_kv_heads, Q = c.num_q_heads, R = c.num_ref, D = c.head_dim;
  const int L = c.levels;
  const int64_t P = (int64_t)mbmax * (Q / H);
  int64_t ncap[MAXL + 1] = {0};
  for (int l = 1; l <= L; ++l) ncap[l] = ceil_div(nodes_at(c, l, c.capacity), 64) * 64;
  a.Qf = (float*)take((size_t)(H * P * D) * 4);
  a.X = (float*)take((size_t)(H * mbmax * (L + 1) * R * (D + 2)) * 4);
  int64_t so = 0, ko = 0;
  for (int l = 1; l <= L; ++l) {
    a.sstride[l] = ncap[l];
    a.soff[l] = so;
    so += H * P * ncap[l];
    a.kstride[l] = ceil_div(ncap[l], 32 * 64) * 64;
    a.koff[l] = ko;
    ko += H * P * a.kstride[l];
  }
  a.S = (float*)take((size_t)so * 4);
  a.KB = (uint32_t*)take((size_t)ko * 4);
  a.L0node = (int32_t*)take((size_t)(mbmax * H * ncap[1]) * 4);
  a.L0mask = (uint32_t*)take((size_t)(mbmax * H * ncap[1]) * 4);
  a.cnt0 = (int32_t*)take((size_t)(mbmax * H) * 4);
  const int ps = (int)std::min<int64_t>(MAX_SPLITS, (int64_t)PF_SPLITS * H);
  float* ap = (float*)take((size_t)(mbmax * Q * ps * (D + 2)) * 4);
  // union attention partials (bf16 caches): [Hkv][P'][splits(P')][D + 2] for every
  // sub-batch size up to mbmax
  int64_t up = 0;
  for (int mb = 1; mb <= mbmax; ++mb) {
    const int64_t pp = (int64_t)mb * (Q / H);
    up = std::max<int64_t>(up, pp * prefill_attend_splits((int)H, (int)pp));
  }
  float* uap = c.dtype == ZHA_BF16 ? (float*)take((size_t)(H * up * (D + 2)) * 4) : nullptr;
  a.mbmax = mbmax;
  if (out) *out = a;
  if (apart) *apart = ap;
  if (pstride) *pstride = ps;
  if (upart) *upart = uap;
  return (off + 255) & ~(size_t)255;
}

}  // namespace

extern "C" {

size_t zha_prefill_workspace_bytes(const zha_config* cfg, int32_t batch) {
  if (validate(cfg) != ZHA_OK || batch < 1 || batch > PF_MAX_BATCH) return 0;
  return prefill_layout(*cfg, batch, nullptr, nullptr, nullptr, nullptr);
}

zha_status zha_prefill_batched(zha_tree* t, const void* k_new, const void* v_new, const void* q, float* out,
                               int64_t m, int32_t batch, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  if (!t) return fail(ZHA_E_INVALID, "tree is null");
  if (!t->built) return fail(ZHA_E_STATE, "prefill before build");
  if (!k_new || !v_new || !q || !out) return fail(ZHA_E_INVALID, "null k_new, v_new, q or out");
  if ((uintptr_t)q % 16) return fail(ZHA_E_INVALID, "q must be 16-byte aligned");
  if (m < 1) return fail(ZHA_E_INVALID, "m %lld < 1", (long long)m);
  if (batch < 1 || batch > PF_MAX_BATCH) return fail(ZHA_E_INVALID, "batch %d outside 1..%d", batch, PF_MAX_BATCH);
  if (!workspace) return fail(ZHA_E_INVALID, "workspace is null");
  if ((uintptr_t)workspace % 256) return fail(ZHA_E_INVALID, "workspace not 256-byte aligned");
  const zha_config& c = t->cfg;
  const size_t need = prefill_layout(c, batch, nullptr, nullptr, nullptr, nullptr);
  if (workspace_bytes < need)
    return fail(ZHA_E_WORKSPACE, "prefill workspace %zu bytes < %zu needed", workspace_bytes, need);
  if (t->N + m > c.capacity)
    return fail(ZHA_E_CAPACITY, "%lld + %lld tokens > capacity %lld", (long long)t->N, (long long)m,
                (long long)c.capacity);
  PrefillArgs a;
  float* apart = nullptr;
  float* upart = nullptr;
  int pstride = 0;
  prefill_layout(c, batch, (char*)workspace, &a, &apart, &pstride, &upart);
  const bool bf16 = c.dtype == ZHA_BF16;
  const int D = c.head_dim, R = c.num_ref, H = c.num_kv_heads, Q = c.num_q_heads, g = Q / H;
  const size_t es = bf16 ? 2 : 4, row = (size_t)D * es;
  a.dev = t->dev;
  a.K = t->K;
  a.V = t->V;
  a.keep_sink = c.keep_sink;
  a.refs = t->refs;
  a.cap = c.capacity;
  a.hkv = H;
  a.hq = Q;
  a.g = g;
  a.b = c.block;
  a.levels = c.levels;
  a.R = R;
  a.D = D;
  a.q_bf16 = bf16 ? 1 : 0;
  a.sigma = 1.0f / sqrtf((float)D);
  for (int l = 0; l <= MAXL; ++l) a.top_p[l] = t->top_p[l];
  const int resident = attend_resident_splits(bf16, D, false, H);
  // attention: the union kernel reads each K/V tile once for all pairs of a sub-batch but
  // each wave reads the tiles its 32 pairs keep, which pays where the heads keep most
  // blocks (level-1 p >= 0.9: deep 256K 0.64 against 0.69 ms, wide 256K 1.0 against 2.1 ms
  // per sub-batch of 32) and not where they keep few (ultra 16M, p 0.75: 24 against 7.5 ms);
  // elsewhere one gather list per query
  const bool union_attn = bf16 && t->top_p[1] >= 0.9f;
  t->pf_valid = false;
  for (int64_t s0 = 0; s0 < m; s0 += batch) {
    const int mb = (int)std::min<int64_t>(batch, m - s0);
    const int64_t N0 = t->N;
    // the sub-batch's tokens: rows s0 .. s0+mb-1 of each KV head's [m][d] chunk
    hipError_t e = hipMemcpy2DAsync((char*)t->K + (size_t)N0 * row, (size_t)c.capacity * row,
                                    (const char*)k_new + (size_t)s0 * row, (size_t)m * row, (size_t)mb * row, H,
                                    hipMemcpyDeviceToDevice, stream);
    if (e == hipSuccess)
      e = hipMemcpy2DAsync((char*)t->V + (size_t)N0 * row, (size_t)c.capacity * row,
                           (const char*)v_new + (size_t)s0 * row, (size_t)m * row, (size_t)mb * row, H,
                           hipMemcpyDeviceToDevice, stream);
    if (e != hipSuccess) return hip_fail(e, "cache row copy");
    zha_status zs = enqueue_build(t, t->K, t->refs, N0, N0 + mb, stream);
    if (zs != ZHA_OK) return zs;
    t->N = N0 + mb;
    a.N0 = N0;
    a.mb = mb;
    a.P = mb * g;
    a.q = (const char*)q + (size_t)s0 * Q * row;
    for (int l = 1; l <= c.levels; ++l) a.nl[l] = nodes_at(c, l, N0 + mb);
    a.nl[0] = a.nl[1];
    {
      ProfScope ps(t, "prefill_prep", stream);
      e = launch_prefill_qprep(a, bf16, D, stream);
      if (e == hipSuccess) e = launch_prefill_prefix(a, bf16, D, R, stream);
    }
    if (e != hipSuccess) return hip_fail(e, "prefill prep launch");
    {
      ProfScope ps(t, "prefill_score", stream);
      e = launch_prefill_score(a, D, R, stream);
      if (e == hipSuccess) e = launch_prefill_tail(a, D, R, stream);
    }
    if (e != hipSuccess) return hip_fail(e, "prefill score launch");
    {
      ProfScope ps(t, "prefill_select", stream);
      e = launch_prefill_select(a, stream);
      if (e == hipSuccess && !union_attn) e = launch_prefill_gather(a, stream);
    }
    if (e != hipSuccess) return hip_fail(e, "prefill select launch");
    t->pf_args = a;
    t->pf_valid = true;
    if (union_attn) {
      // the union attention over the kept bitmaps
      ProfScope ps(t, "prefill_attend", stream);
      e = launch_prefill_attend(a, upart, out + (size_t)s0 * Q * D, D, stream);
      if (e != hipSuccess) return hip_fail(e, "prefill attention launch");
      continue;
    }
    AttnArgs at;
    memset(&at, 0, sizeof at);
    at.dev = t->dev;
    at.dev.node[0] = a.L0node;
    at.dev.mask[0] = a.L0mask;
    at.dev.cnt = a.cnt0;
    at.dev.apart = apart;
    at.K = t->K;
    at.V = t->V;
    at.q = a.q;
    at.cap = c.capacity;
    at.N = N0 + 1;
    at.n_step = 1;
    at.hkv = H;
    at.hq = Q;
    at.g = g;
    at.b = c.block;
    at.splits = std::max(1, std::min(PF_SPLITS, resident / mb));
    at.pstride = pstride;
    at.keep_sink = c.keep_sink;
    at.sigma = a.sigma;
    at.out = out + (size_t)s0 * Q * D;
    at.q_stride = (int64_t)Q * D;
    at.l_stride = (int64_t)H * t->dev.ncap[1];
    at.p_stride = (int64_t)Q * pstride * (D + 2);
    at.o_stride = (int64_t)Q * D;
    at.c_stride = H;
    {
      ProfScope ps(t, "prefill_attend", stream);
      e = launch_attend_batch(at, bf16, D, mb, stream);
    }
    if (e != hipSuccess) return hip_fail(e, "prefill attention launch");
  }
  return ZHA_OK;
}

zha_status zha_debug_prefill_trace(zha_tree* t, int32_t level, float* scores, uint32_t* kept, float* own,
                                   hipStream_t stream) {
  if (!t) return fail(ZHA_E_INVALID, "tree is null");
  if (!t->pf_valid) return fail(ZHA_E_STATE, "no batched prefill to trace");
  const PrefillArgs& a = t->pf_args;
  if (level < 1 || level > a.levels) return fail(ZHA_E_INVALID, "level %d outside 1..%d", level, a.levels);
  const int64_t n = a.nl[level], nw = (n + 31) >> 5, rows = (int64_t)a.hkv * a.P;
  hipError_t e = hipSuccess;
  if (scores)
    e = hipMemcpy2DAsync(scores, (size_t)n * 4, a.S + a.soff[level], (size_t)a.sstride[level] * 4, (size_t)n * 4,
                         (size_t)rows, hipMemcpyDeviceToDevice, stream);
  if (e == hipSuccess && kept)
    e = hipMemcpy2DAsync(kept, (size_t)nw * 4, a.KB + a.koff[level], (size_t)a.kstride[level] * 4, (size_t)nw * 4,
                         (size_t)rows, hipMemcpyDeviceToDevice, stream);
  const int64_t node = (int64_t)a.R * (a.D + 2);
  for (int kv = 0; own && e == hipSuccess && kv < a.hkv; ++kv)
    e = hipMemcpy2DAsync(own + (int64_t)kv * a.mb * node, (size_t)node * 4,
                         a.X + ((int64_t)kv * a.mbmax * (a.levels + 1) + level) * node,
                         (size_t)(a.levels + 1) * node * 4, (size_t)node * 4, (size_t)a.mb, hipMemcpyDeviceToDevice,
                         stream);
  if (e != hipSuccess) return hip_fail(e, "prefill trace copy");
  return ZHA_OK;
}

zha_status zha_decode_dense(zha_tree* t, const void* q, float* out, hipStream_t stream) {
  if (!t) return fail(ZHA_E_INVALID, "tree is null");
  if (!t->built) return fail(ZHA_E_STATE, "decode before build");
  if (!q || !out) return fail(ZHA_E_INVALID, "null q or out");
  if ((uintptr_t)q % 16) return fail(ZHA_E_INVALID, "q must be 16-byte aligned");
  const zha_config& c = t->cfg;
  AttnArgs a;
  memset(&a, 0, sizeof a);
  a.dev = t->dev;
  a.K = t->K;
  a.V = t->V;
  a.q = q;
  a.cap = c.capacity;
  a.N = t->N;
  a.hkv = c.num_kv_heads;
  a.hq = c.num_q_heads;
  a.g = a.hq / a.hkv;
  a.b = c.block;
  a.splits = attn_splits(t->N, 1024, attend_resident_splits(c.dtype == ZHA_BF16, c.head_dim, true, c.num_kv_heads));
  a.keep_sink = 0;
  a.pstride = MAX_SPLITS;
  a.sigma = 1.0f / sqrtf((float)c.head_dim);
  a.out = out;
  hipError_t e;
  {
    ProfScope ps(t, "dense_attend", stream);
    e = launch_attend(a, c.dtype == ZHA_BF16, c.head_dim, true, stream);
  }
  if (e != hipSuccess) return hip_fail(e, "dense attention launch");
  return ZHA_OK;
}

}  // extern "C"

// Scratch of the allocation-free dense decode: the split-K attention partials
// [Hq][splits][D + 2] in a fixed array, one copy per GPU, held until the process ends.  Host
// code never passes the array's name to a kernel: it takes the device address from
// hipGetSymbolAddress once per device (with that device current) and uses that.
constexpr size_t STATIC_SCRATCH_BYTES = (size_t)4 << 20;
static __device__ __align__(256) float scratch[STATIC_SCRATCH_BYTES / 4];

namespace {

constexpr int SCRATCH_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[SCRATCH_MAX_DEVICES];

// Device address of the current device's scratch array.
zha_status scratch_for_current_device(float** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "current device");
  if (dev < 0 || dev >= SCRATCH_MAX_DEVICES)
    return fail(ZHA_E_UNSUPPORTED, "device %d: the static scratch serves devices 0..%d", dev, SCRATCH_MAX_DEVICES - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "static scratch address");
    if (!p) return fail(ZHA_E_HIP, "static scratch address is null");
    g_scratch_ptr[dev] = (float*)p;
  }
  *out = g_scratch_ptr[dev];
  return ZHA_OK;
}

}  // namespace

extern "C" {

zha_status zha_decode_dense_static(const zha_config* cfg, const void* k_cache, const void* v_cache, int64_t n_tokens,
                                   const void* q, float* out, hipStream_t stream) {
  zha_status s = validate(cfg);
  if (s != ZHA_OK) return s;
  if (!k_cache || !v_cache || !q || !out) return fail(ZHA_E_INVALID, "null cache, q or out");
  if (((uintptr_t)k_cache | (uintptr_t)v_cache | (uintptr_t)q) % 16)
    return fail(ZHA_E_INVALID, "cache and q pointers must be 16-byte aligned");
  if (n_tokens < 1) return fail(ZHA_E_INVALID, "n_tokens %lld < 1", (long long)n_tokens);
  if (n_tokens > cfg->capacity)
    return fail(ZHA_E_CAPACITY, "n_tokens %lld > capacity %lld", (long long)n_tokens, (long long)cfg->capacity);
  const zha_config& c = *cfg;
  // one split's partials over every query head; the splits per KV head are capped so that
  // all partials fit the static array
  const size_t per_split = (size_t)c.num_q_heads * (size_t)(c.head_dim + 2) * 4;
  const int64_t fit = (int64_t)(STATIC_SCRATCH_BYTES / per_split);
  if (fit < 1)
    return fail(ZHA_E_WORKSPACE, "%d query heads of head_dim %d need %zu bytes of partials, above the %zu-byte static scratch",
                c.num_q_heads, c.head_dim, per_split, STATIC_SCRATCH_BYTES);
  float* sp = nullptr;
  s = scratch_for_current_device(&sp);
  if (s != ZHA_OK) return s;
  AttnArgs a;
  memset(&a, 0, sizeof a);
  a.dev.apart = sp;
  a.K = k_cache;
  a.V = v_cache;
  a.q = q;
  a.cap = c.capacity;
  a.N = n_tokens;
  a.hkv = c.num_kv_heads;
  a.hq = c.num_q_heads;
  a.g = a.hq / a.hkv;
  a.b = c.block;
  const int resident = attend_resident_splits(c.dtype == ZHA_BF16, c.head_dim, true, c.num_kv_heads);
  a.splits = attn_splits(n_tokens, 1024, (int)(fit < resident ? fit : resident));
  a.pstride = a.splits;
  a.keep_sink = 0;
  a.sigma = 1.0f / sqrtf((float)c.head_dim);
  a.out = out;
  hipError_t e = launch_attend(a, c.dtype == ZHA_BF16, c.head_dim, true, stream);
  if (e != hipSuccess) return hip_fail(e, "dense attention launch");
  return ZHA_OK;
}

zha_status zha_debug_level(zha_tree* t, int32_t level, float* s_out, float* c_out, hipStream_t stream) {
  if (!t) return fail(ZHA_E_INVALID, "tree is null");
  if (!t->built) return fail(ZHA_E_STATE, "no tree built");
  if (level < 1 || level > t->cfg.levels) return fail(ZHA_E_INVALID, "level %d outside 1..%d", level, t->cfg.levels);
  if (!s_out || !c_out) return fail(ZHA_E_INVALID, "null output");
  const zha_config& c = t->cfg;
  const int64_t n = nodes_at(c, level, t->N), cap = t->dev.ncap[level];
  const size_t srow = (size_t)c.num_ref * c.head_dim * 4, crow = (size_t)c.num_ref * 4;
  for (int kv = 0; kv < c.num_kv_heads; ++kv) {
    hipError_t e = hipMemcpyAsync((char*)s_out + kv * n * srow, (char*)t->dev.s[level] + kv * cap * srow, n * srow,
                                  hipMemcpyDeviceToDevice, stream);
    if (e == hipSuccess)
      e = hipMemcpyAsync((char*)c_out + kv * n * crow, (char*)t->dev.c[level] + kv * cap * crow, n * crow,
                         hipMemcpyDeviceToDevice, stream);
    if (e != hipSuccess) return hip_fail(e, "level copy");
  }
  return ZHA_OK;
}

zha_status zha_debug_router_planes(zha_tree* t, int32_t level, void* s_out, void* scale_out, hipStream_t stream) {
  if (!t) return fail(ZHA_E_INVALID, "tree is null");
  if (!t->built) return fail(ZHA_E_STATE, "no tree built");
  if (level < 1 || level > t->cfg.levels) return fail(ZHA_E_INVALID, "level %d outside 1..%d", level, t->cfg.levels);
  if (!s_out) return fail(ZHA_E_INVALID, "null output");
  const bool fp4 = t->dev.s4[level] != nullptr;
  if (!t->dev.sq[level] && !fp4) return fail(ZHA_E_INVALID, "no quantised router planes at level %d", level);
  if (fp4 && !scale_out) return fail(ZHA_E_INVALID, "null scale output");
  const zha_config& c = t->cfg;
  const int64_t n = nodes_at(c, level, t->N), cap = t->dev.ncap[level];
  const size_t rd = (size_t)c.num_ref * c.head_dim;
  const size_t srow = fp4 ? rd / 2 : rd * 2, xrow = rd / 32;
  const char* src = fp4 ? (const char*)t->dev.s4[level] : (const char*)t->dev.sq[level];
  for (int kv = 0; kv < c.num_kv_heads; ++kv) {
    hipError_t e = hipMemcpyAsync((char*)s_out + kv * n * srow, src + kv * cap * srow, n * srow,
                                  hipMemcpyDeviceToDevice, stream);
    if (e == hipSuccess && fp4)
      e = hipMemcpyAsync((char*)scale_out + kv * n * xrow, (const char*)t->dev.s4x[level] + kv * cap * xrow, n * xrow,
                         hipMemcpyDeviceToDevice, stream);
    if (e != hipSuccess) return hip_fail(e, "router plane copy");
  }
  return ZHA_OK;
}

zha_status zha_debug_trace(zha_tree* t, int32_t level, int64_t cap, int32_t* nodes, uint32_t* masks, float* scores,
                           uint32_t* keep, int32_t* counts, hipStream_t stream) {
  if (!t) return fail(ZHA_E_INVALID, "tree is null");
  if (!t->built) return fail(ZHA_E_STATE, "no tree built");
  const zha_config& c = t->cfg;
  if (level < 0 || level > c.levels) return fail(ZHA_E_INVALID, "level %d outside 0..%d", level, c.levels);
  if (!nodes || !masks || !counts) return fail(ZHA_E_INVALID, "null output");
  const int64_t n = nodes_at(c, level == 0 ? 1 : level, t->N);
  if (cap < n) return fail(ZHA_E_INVALID, "cap %lld < %lld nodes", (long long)cap, (long long)n);
  const int64_t dcap = t->dev.ncap[level];
  hipError_t e = hipSuccess;
  if (t->td_valid && !t->td_lists && level >= t->td_args.dense_lo && level <= t->td_args.level) {
    // the dense union lists of the last top-down selection, from its bitmaps
    e = launch_route_td_lists(t->td_args, stream);
    if (e != hipSuccess) return hip_fail(e, "top-down list launch");
    t->td_lists = true;
  }
  for (int kv = 0; kv < c.num_kv_heads && e == hipSuccess; ++kv) {
    e = hipMemcpyAsync(nodes + kv * cap, t->dev.node[level] + kv * dcap, n * 4, hipMemcpyDeviceToDevice, stream);
    if (e == hipSuccess)
      e = hipMemcpyAsync(masks + kv * cap, t->dev.mask[level] + kv * dcap, n * 4, hipMemcpyDeviceToDevice, stream);
    if (e == hipSuccess && keep && level >= 1)
      e = hipMemcpyAsync(keep + kv * cap, t->dev.keep[level] + kv * dcap, n * 4, hipMemcpyDeviceToDevice, stream);
    for (int gi = 0; gi < GMAX && e == hipSuccess && scores && level >= 1; ++gi)
      e = hipMemcpyAsync(scores + ((int64_t)kv * GMAX + gi) * cap, t->dev.score[level] + ((int64_t)kv * GMAX + gi) * dcap,
                         n * 4, hipMemcpyDeviceToDevice, stream);
  }
  if (e == hipSuccess)
    e = hipMemcpyAsync(counts, t->dev.cnt + (int64_t)level * c.num_kv_heads, c.num_kv_heads * 4,
                       hipMemcpyDeviceToDevice, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "trace copy");
  return ZHA_OK;
}

zha_status zha_debug_route_level(zha_tree* t, int32_t level, const void* q, const int32_t* nodes,
                                 const uint32_t* masks, const int32_t* counts, int64_t cap, int32_t path,
                                 hipStream_t stream) {
  if (!t) return fail(ZHA_E_INVALID, "tree is null");
  if (!t->built) return fail(ZHA_E_STATE, "no tree built");
  const zha_config& c = t->cfg;
  if (level < 1 || level > c.levels) return fail(ZHA_E_INVALID, "level %d outside 1..%d", level, c.levels);
  if (!q || !nodes || !masks || !counts) return fail(ZHA_E_INVALID, "null input");
  if (path != 0 && path != 1) return fail(ZHA_E_INVALID, "path %d is neither 0 nor 1", path);
  const int64_t n = nodes_at(c, level, t->N);
  const int H = c.num_kv_heads;
  std::vector<int32_t> hc(H);
  hipError_t e = hipMemcpyAsync(hc.data(), counts, H * 4, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "count read");
  for (int kv = 0; kv < H; ++kv) {
    if (hc[kv] < 0 || hc[kv] > n || hc[kv] > cap)
      return fail(ZHA_E_INVALID, "count %d for KV head %d outside 0..%lld", hc[kv], kv, (long long)n);
    std::vector<int32_t> hn(hc[kv]);
    if (hc[kv]) {
      e = hipMemcpy(hn.data(), nodes + kv * cap, hc[kv] * 4, hipMemcpyDeviceToHost);
      if (e != hipSuccess) return hip_fail(e, "node read");
    }
    for (int i = 0; i < hc[kv]; ++i)
      if (hn[i] < 0 || hn[i] >= n || (i && hn[i] <= hn[i - 1]))
        return fail(ZHA_E_INVALID, "node list of KV head %d not ascending in 0..%lld", kv, (long long)n - 1);
  }
  RouteArgs r = route_args(t, q);
  r.nlevel = nodes_at(c, c.levels, t->N);
  e = launch_route_prep(r, c.dtype == ZHA_BF16, c.head_dim, stream);
  if (e != hipSuccess) return hip_fail(e, "route prep launch");
  const int64_t dcap = t->dev.ncap[level];
  for (int kv = 0; kv < H && e == hipSuccess; ++kv) {
    if (!hc[kv]) continue;
    e = hipMemcpyAsync(t->dev.node[level] + kv * dcap, nodes + kv * cap, hc[kv] * 4, hipMemcpyDeviceToDevice, stream);
    if (e == hipSuccess)
      e = hipMemcpyAsync(t->dev.mask[level] + kv * dcap, masks + kv * cap, hc[kv] * 4, hipMemcpyDeviceToDevice,
                         stream);
  }
  if (e == hipSuccess)
    e = hipMemcpyAsync(t->dev.cnt + (int64_t)level * H, counts, H * 4, hipMemcpyDeviceToDevice, stream);
  if (e != hipSuccess) return hip_fail(e, "frontier copy");
  if (path == 0 && r.allkeys) {
    // the decode's kernels: every node scored from the keys, the top-down selection of this
    // level started from the given per-head frontiers, the dense union list
    r.level = level;
    r.dense_lo = level;
    r.nlevel = r.nl[level];
    e = launch_route_td_seed(r, stream);
    if (e != hipSuccess) return hip_fail(e, "frontier seed launch");
    e = launch_route_allkeys_score(r, c.head_dim, c.num_ref, stream);
    if (e != hipSuccess) return hip_fail(e, "route key score launch");
    r.tf = 1;
    e = launch_route_topdown_keys(r, stream);
    if (e == hipSuccess) e = launch_route_td_lists(r, stream);
    if (e != hipSuccess) return hip_fail(e, "route top-down select launch");
    t->td_args = r;
    t->td_valid = true;
    t->td_lists = true;
  } else if (path == 0 && level >= topdown_lo(r)) {
    // the decode's kernels for this level: every node scored, the top-down selection
    // started from the given per-head frontiers, the dense union list
    r.level = level;
    r.dense_lo = level;
    r.nlevel = r.nl[level];
    e = launch_route_td_seed(r, stream);
    if (e != hipSuccess) return hip_fail(e, "frontier seed launch");
    r.dense = 1;
    e = launch_route_dense_score(r, c.head_dim, c.num_ref, stream);
    if (e != hipSuccess) return hip_fail(e, "route dense score launch");
    r.dense = 0;
    r.tf = 1;
    e = launch_route_topdown(r, stream);
    if (e == hipSuccess) e = launch_route_td_lists(r, stream);
    if (e != hipSuccess) return hip_fail(e, "route top-down select launch");
    t->td_args = r;
    t->td_valid = true;
    t->td_lists = true;
  } else {
    t->td_valid = false;
    zha_status zs = route_levels(t, r, level, stream, false);
    if (zs != ZHA_OK) return zs;
  }
  e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "route level");
  return ZHA_OK;
}

zha_status zha_set_top_p_levels(zha_tree* t, const float* p_levels) {
  if (!t) return fail(ZHA_E_INVALID, "tree is null");
  const int L = t->cfg.levels;
  if (p_levels)
    for (int l = 0; l < L; ++l)
      if (!(p_levels[l] > 0.f && p_levels[l] <= 1.f))
        return fail(ZHA_E_INVALID, "p of level %d is %g, outside (0, 1]", l + 1, p_levels[l]);
  for (int l = 1; l <= L; ++l) t->top_p[l] = p_levels ? p_levels[l - 1] : t->cfg.top_p;
  return ZHA_OK;
}

zha_status zha_debug_check(zha_tree* t, uint32_t* flags, hipStream_t stream) {
  if (!t) return fail(ZHA_E_INVALID, "tree is null");
  if (!flags) return fail(ZHA_E_INVALID, "flags is null");
  uint32_t v = 0;
  hipError_t e = hipMemcpyAsync(&v, t->dev.err, 4, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e == hipSuccess) e = hipMemsetAsync(t->dev.err, 0, 4, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "check word");
  *flags = v;
  return ZHA_OK;
}

int32_t zha_debug_checks_compiled(void) {
#ifdef ZHA_DEBUG
  return 1;
#else
  return 0;
#endif
}

int64_t zha_num_tokens(const zha_tree* t) { return t ? t->N : -1; }

zha_status zha_profile_start(zha_tree* t, const char* key_prefix) {
  if (!t) return fail(ZHA_E_INVALID, "tree is null");
  if (!key_prefix) return fail(ZHA_E_INVALID, "key prefix is null");
  if (t->prof.on) return fail(ZHA_E_STATE, "profiling already active");
  t->prof.on = true;
  t->prof.prefix = key_prefix;
  t->prof.ev.clear();
  return ZHA_OK;
}

zha_status zha_profile_stop(zha_tree* t, double* total_ms, int64_t* launches) {
  if (!t) return fail(ZHA_E_INVALID, "tree is null");
  if (!t->prof.on) return fail(ZHA_E_STATE, "profiling not active");
  double tot = 0.0;
  hipError_t err = hipSuccess;
  for (auto& pr : t->prof.ev) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(pr.second);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, pr.first, pr.second);
    if (e != hipSuccess && err == hipSuccess) err = e;
    tot += ms;
    (void)hipEventDestroy(pr.first);
    (void)hipEventDestroy(pr.second);
  }
  const int64_t n = (int64_t)t->prof.ev.size();
  t->prof.ev.clear();
  t->prof.on = false;
  if (err != hipSuccess) return hip_fail(err, "profile events");
  if (total_ms) *total_ms = tot;
  if (launches) *launches = n;
  return ZHA_OK;
}

zha_status zha_destroy(zha_tree* t) {
  if (!t) return fail(ZHA_E_INVALID, "tree is null");
  for (auto& pr : t->prof.ev) {
    (void)hipEventDestroy(pr.first);
    (void)hipEventDestroy(pr.second);
  }
  delete t;
  return ZHA_OK;
}

const char* zha_status_string(zha_status s) {
  switch (s) {
    case ZHA_OK: return "ok";
    case ZHA_E_INVALID: return "invalid argument";
    case ZHA_E_UNSUPPORTED: return "unsupported configuration";
    case ZHA_E_CAPACITY: return "capacity exceeded";
    case ZHA_E_WORKSPACE: return "workspace too small";
    case ZHA_E_STATE: return "call out of order";
    case ZHA_E_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* zha_last_error(void) { return g_err.c_str(); }

}  // extern "C"
