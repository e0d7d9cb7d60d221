"""Plain, slow CPU oracle of the ZHA decode hot path.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import or run this module.  The product path (the HIP library and its Python binding)
never imports it and shares no code with it.

Everything is NumPy in float64 on the exact values of the (fp32 or bf16) inputs.  Each
function follows the method as the pages describe it; where a step is open the reading
taken is stated in the function's docstring.

Sources (all about Zyphra Hierarchical Attention, arXiv 2610.42112):
  [blog]  Zyphra's blog post "Zyphra Hierarchical Attention" (translated copies), sections
          "Building the tree", "Routing through the tree", "How is this subquadratic".
  [news]  news summary "Zyphra releases the ZHA sparse attention method" (tanhow.com),
          sections "Building the tree" and "How does top-p routing pick tokens?".
  [abs]   the paper's abstract "Subquadratic Attention with a Hierarchical
          Tree-Structured Indexer".

Notation: d = head dim, sigma = 1/sqrt(d), b = block, R reference queries r_j,
level-l node n spans tokens [n*b^l, min((n+1)*b^l, N)).

Parity pins: every function here is pinned by the CPU tests in ``tests/test_oracle_pins.py``
(dense limit at p=1, convexity lower bound, exactness at q=r_j, recursion = direct
per-span form, single-key blocks, nucleus selection for b=1, brute-force minimality,
mass conservation, append = rebuild, geometry; for the bf16 router planes: rounding
against torch's float32 -> bfloat16 cast and a brute-force nearest search, and the score
perturbation bound; for FP4 planes: a brute-force nearest search over the 16 codes,
constructed halfway cases, the block-scale property and the same bound; for the
reference-query fit: central differences of the loss, the exact level-1 router of
single-key blocks, non-negativity and a brute-force loss).  The exact
routed sets at p<1 on the synthetic data are defined only by this oracle ("parity
unpinned" beyond those pins).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


def _logsumexp(x: np.ndarray, axis: int) -> np.ndarray:
    """log(sum(exp(x))) along ``axis``; -inf where every entry is -inf."""
    m = np.max(x, axis=axis, keepdims=True)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    with np.errstate(divide="ignore"):
        out = np.log(np.sum(np.exp(x - m_safe), axis=axis, keepdims=True)) + m_safe
    return np.squeeze(out, axis=axis)


# --------------------------------------------------------------------------- tree build
def level1_planes(keys: np.ndarray, refs: np.ndarray, block: int) -> tuple[np.ndarray, np.ndarray]:
    """Level-1 summaries: one tangent plane per block and reference query.

    [news] "Building the tree": keys are cut into contiguous blocks and each reference
    query gives a tangent-plane estimate of the block's log attention mass.  For block B
    and query r_j the log mass is f(q) = log sum_{k in B} exp(sigma q.k); its tangent
    plane at q = r_j has gradient sigma * s_j with s_j = sum_k softmax_k(sigma r_j.k) k
    (the softmax-weighted mean key) and value LSE_j = f(r_j).  We store the plane as
    (s_j, c_j) with c_j = LSE_j - sigma r_j.s_j, so plane_j(q) = sigma q.s_j + c_j and
    plane_j(r_j) = LSE_j.  The last block may be partial (only tokens < N exist).

    keys [N, d], refs [R, d]  ->  s [n1, R, d], c [n1, R]
    """
    keys = np.asarray(keys, dtype=np.float64)
    refs = np.asarray(refs, dtype=np.float64)
    n, d = keys.shape
    sig = 1.0 / math.sqrt(d)
    n1 = -(-n // block)
    padded = np.zeros((n1 * block, d))
    padded[:n] = keys
    kb = padded.reshape(n1, block, d)
    exists = (np.arange(n1 * block) < n).reshape(n1, block)
    z = sig * (kb @ refs.T)                                   # [n1, b, R]
    z = np.where(exists[:, :, None], z, -np.inf)
    lse = _logsumexp(z, axis=1)                               # [n1, R]
    w = np.exp(z - lse[:, None, :])                           # softmax over the block's keys
    s = np.transpose(w, (0, 2, 1)) @ kb                       # [n1, R, d] weighted mean keys
    c = lse - sig * np.sum(s * refs[None, :, :], axis=2)
    return s, c


def parent_planes(s_child: np.ndarray, c_child: np.ndarray, refs: np.ndarray,
                  block: int) -> tuple[np.ndarray, np.ndarray]:
    """Summaries one level up, built from the children's planes only.

    [blog] "Building the tree" / [abs]: summaries are grouped b at a time and compressed
    again, recursively.  Parent n has children n*b .. n*b+b-1 (those that exist).  For
    each child c and reference query r_j, the child's estimate at r_j is its router score
    there, e_cj = max_i(sigma r_j.s_ci + c_ci), attained by plane i* (lowest index on a
    tie).  The parent's log mass at r_j is LSE_j = logsumexp_c e_cj, its gradient is the
    children's weighted mean sum_c softmax_c(e_cj) * s_{c,i*} (the gradient of each
    child's max is its arg-max plane), and c_j = LSE_j - sigma r_j.s_j as at level 1.

    s_child [nc, R, d], c_child [nc, R]  ->  s [np, R, d], c [np, R]
    """
    s_child = np.asarray(s_child, dtype=np.float64)
    c_child = np.asarray(c_child, dtype=np.float64)
    refs = np.asarray(refs, dtype=np.float64)
    nc, r, d = s_child.shape
    sig = 1.0 / math.sqrt(d)
    npar = -(-nc // block)
    # est[c, j, i] = plane i of child c evaluated at reference query j
    est = sig * np.transpose(s_child @ refs.T, (0, 2, 1)) + c_child[:, None, :]
    istar = np.argmax(est, axis=2)                            # [nc, R] (first max on ties)
    e = np.take_along_axis(est, istar[:, :, None], axis=2)[:, :, 0]
    grad = np.take_along_axis(s_child, istar[:, :, None], axis=1)   # [nc, R, d]
    e_pad = np.full((npar * block, r), -np.inf)
    e_pad[:nc] = e
    g_pad = np.zeros((npar * block, r, d))
    g_pad[:nc] = grad
    e_pad = e_pad.reshape(npar, block, r)
    g_pad = g_pad.reshape(npar, block, r, d)
    lse = _logsumexp(e_pad, axis=1)                           # [np, R]
    w = np.exp(e_pad - lse[:, None, :])                       # softmax over children
    s = np.sum(w[:, :, :, None] * g_pad, axis=1)              # [np, R, d]
    c = lse - sig * np.sum(s * refs[None, :, :], axis=2)
    return s, c


@dataclasses.dataclass
class Tree:
    """One KV head's tree over keys[:n_tokens]: levels[l-1] = (s, c) of level l."""
    keys: np.ndarray          # [capacity, d] float64 (rows >= n_tokens unused until appended)
    refs: np.ndarray          # [R, d] float64
    block: int
    n_levels: int
    n_tokens: int
    levels: list

    def nodes(self, level: int) -> int:
        return -(-self.n_tokens // self.block ** level)


def build_tree(keys: np.ndarray, refs: np.ndarray, block: int, levels: int, n_tokens: int) -> Tree:
    """Level 1 from the raw keys, then each level from the one below it."""
    keys = np.asarray(keys, dtype=np.float64)
    out = [level1_planes(keys[:n_tokens], refs, block)]
    for _ in range(2, levels + 1):
        out.append(parent_planes(out[-1][0], out[-1][1], refs, block))
    return Tree(keys=keys, refs=np.asarray(refs, dtype=np.float64), block=block, n_levels=levels,
                n_tokens=n_tokens, levels=out)


def append_token(tree: Tree, key: np.ndarray) -> None:
    """Add token N and refresh the one node per level whose span now contains it.

    The pages say nothing about incremental updates; appending is the decode-time
    counterpart of the build.  Only the rightmost node of each level covers the new
    token, so that node is recomputed from its keys (level 1) or its children; a level
    gains a node when N crosses a multiple of b^l.
    """
    n = tree.n_tokens
    tree.keys[n] = np.asarray(key, dtype=np.float64)
    tree.n_tokens = n + 1
    b = tree.block
    for lv in range(1, tree.n_levels + 1):
        node = n // b ** lv
        if lv == 1:
            s, c = level1_planes(tree.keys[node * b:min((node + 1) * b, n + 1)], tree.refs, b)
        else:
            sc, cc = tree.levels[lv - 2]
            s, c = parent_planes(sc[node * b:(node + 1) * b], cc[node * b:(node + 1) * b], tree.refs, b)
        s_all, c_all = tree.levels[lv - 1]
        if node == s_all.shape[0]:
            s_all = np.concatenate([s_all, s], axis=0)
            c_all = np.concatenate([c_all, c], axis=0)
        else:
            s_all = s_all.copy()
            c_all = c_all.copy()
            s_all[node] = s[0]
            c_all[node] = c[0]
        tree.levels[lv - 1] = (s_all, c_all)


# --------------------------------------------------------------------------- reference-query fitting
def node_log_mass(keys: np.ndarray, q: np.ndarray, block: int, level: int, n_tokens: int) -> np.ndarray:
    """Dense attention mass of each level-``level`` node for query q, as a log.

    [news] "How is ZHA trained onto existing models?": the fitting target is the dense
    attention mass of every block at every level.  With z_t = sigma q.k_t over all
    n_tokens keys, node n holds tokens [n b^l, (n+1) b^l) and its mass is
    sum over those tokens of softmax(z)_t.  Returns log mass [n_l].
    """
    keys = np.asarray(keys, dtype=np.float64)[:n_tokens]
    q = np.asarray(q, dtype=np.float64)
    span = block ** level
    nn = -(-n_tokens // span)
    z = (keys @ q) / math.sqrt(q.shape[0])
    zp = np.full(nn * span, -np.inf)
    zp[:n_tokens] = z
    return _logsumexp(zp.reshape(nn, span), axis=1) - _logsumexp(z, axis=0)


def router_log_probs(tree: Tree, level: int, q: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """The router's estimated distribution over all nodes of a level for query q:
    softmax of the node scores max_j(sigma q.s_j + c_j) over the level ([blog] "Routing
    through the tree": the scores are estimates of each node's log attention mass).
    Returns (log probabilities [n_l], arg-max plane [n_l], lowest index on a tie)."""
    s, c = tree.levels[level - 1]
    q = np.asarray(q, dtype=np.float64)
    f = (s @ q) / math.sqrt(q.shape[0]) + c                   # [n_l, R]
    am = np.argmax(f, axis=1)
    sc = f[np.arange(f.shape[0]), am]
    return sc - _logsumexp(sc, axis=0), am


def fit_loss(keys: np.ndarray, refs: np.ndarray, block: int, levels: int, n_tokens: int,
             queries: np.ndarray) -> float:
    """KL fitting loss of the reference queries of one tree.

    [blog] "Routing through the tree" and [news] "How is ZHA trained onto existing
    models?": the model stays frozen and only the reference queries are trained, so that
    at every level of the tree the router's probabilities reproduce how dense attention
    spreads its mass over the nodes.  Readings: the divergence is KL(dense || router)
    over all nodes of a level (the distillation direction: the dense mass is the target),
    summed over the levels and averaged over the training queries; the tree is rebuilt
    from the reference queries as in ``build_tree``.

    queries [Q, d] (the training queries of the KV head's group)  ->  loss
    """
    tree = build_tree(keys, refs, block, levels, n_tokens)
    total = 0.0
    for q in np.asarray(queries, dtype=np.float64):
        for lv in range(1, levels + 1):
            logm = node_log_mass(keys, q, block, lv, n_tokens)
            logpi, _ = router_log_probs(tree, lv, q)
            m = np.exp(logm)
            total += float(np.sum(np.where(m > 0, m * (logm - logpi), 0.0)))
    return total / len(queries)


def fit_grad(keys: np.ndarray, refs: np.ndarray, block: int, levels: int, n_tokens: int,
             queries: np.ndarray) -> tuple[float, np.ndarray]:
    """``fit_loss`` and its gradient with respect to the reference queries.

    Node n's score for q is plane i*(q, n) at q (the arg-max plane; its gradient is the
    subgradient of the max).  The plane of reference query r over the node's tokens is
    LSE(r) + sigma (q - r).s(r), with s(r) = sum_t softmax_t(sigma r.k_t) k_t, so its
    derivative in r is sigma^2 C (q - r) with C = sum_t w_t (k_t - s)(k_t - s)^T the
    covariance of the node's keys under those weights.  The derivative of KL(m || pi) in
    the node's score is pi - m.  Returns (loss, grad [R, d]).
    """
    keys = np.asarray(keys, dtype=np.float64)
    refs = np.asarray(refs, dtype=np.float64)
    queries = np.asarray(queries, dtype=np.float64)
    d = keys.shape[1]
    sig = 1.0 / math.sqrt(d)
    tree = build_tree(keys, refs, block, levels, n_tokens)
    grad = np.zeros_like(refs)
    total = 0.0
    for lv in range(1, levels + 1):
        span = block ** lv
        nn = tree.nodes(lv)
        kp = np.zeros((nn * span, d))
        kp[:n_tokens] = keys[:n_tokens]
        kn = kp.reshape(nn, span, d)                          # the keys of each node
        exists = (np.arange(nn * span) < n_tokens).reshape(nn, span)
        s, _ = tree.levels[lv - 1]
        for q in queries:
            logm = node_log_mass(keys, q, block, lv, n_tokens)
            logpi, am = router_log_probs(tree, lv, q)
            m = np.exp(logm)
            total += float(np.sum(np.where(m > 0, m * (logm - logpi), 0.0)))
            g = np.exp(logpi) - m                             # d KL / d score
            r = refs[am]                                      # [nn, d] each node's arg-max query
            zr = sig * np.einsum("ntd,nd->nt", kn, r)
            zr = np.where(exists, zr, -np.inf)
            w = np.exp(zr - _logsumexp(zr, axis=1)[:, None])  # [nn, span]
            diff = kn - s[np.arange(nn), am][:, None, :]      # k_t - s
            a = np.einsum("ntd,nd->nt", diff, q[None, :] - r)
            contrib = sig * sig * np.einsum("nt,ntd->nd", w * a, diff) * g[:, None]
            np.add.at(grad, am, contrib)
    return total / len(queries), grad / len(queries)


# --------------------------------------------------------------------------- bf16 router planes
def bf16_round(x: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 value of each element, as float64 (normal range).

    bfloat16 keeps 8 significant bits (the float32 exponent range, a 7-bit stored
    mantissa); a value halfway between two neighbours goes to the one with an even last
    bit.  Written from that definition: with x = m * 2^e and 1/2 <= |m| < 1, the kept
    value is round(m * 2^8) * 2^(e-8), np.round rounding halves to even.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.round(np.ldexp(m, 8)), e - 8)


E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])   # FP4 magnitudes, codes 0..7
MX_BLOCK = 32


def mxfp4_round(x: np.ndarray, scale_exp=None) -> np.ndarray:
    """OCP MX FP4 round trip of each row (last axis, a multiple of 32 long), as float64.

    Each block of 32 consecutive elements shares a power-of-two scale X = 2^(floor(log2
    amax) - 2), amax the block's largest magnitude and 2 the largest exponent of the E2M1
    element format (largest value 6 = 1.5 * 2^2), so amax / X lies in [4, 8).  Each element
    becomes the nearest of X * {0, 0.5, 1, 1.5, 2, 3, 4, 6} with its sign; a value halfway
    between two of them takes the one whose mantissa bit is 0 (code even); magnitudes above
    6X become 6X.  An all-zero block stays zero.  ``scale_exp`` (one integer per block)
    imposes log2 X instead (the comparison tests use it to bound the result when a block's
    amax sits at a power of two).
    """
    x = np.asarray(x, dtype=np.float64)
    xb = x.reshape(-1, MX_BLOCK)
    amax = np.max(np.abs(xb), axis=1)
    _, e = np.frexp(amax)                       # amax = m * 2^e, 1/2 <= m < 1
    if scale_exp is None:
        scale = np.where(amax > 0, np.ldexp(1.0, e - 1 - 2), 1.0)[:, None]
    else:
        scale = np.ldexp(1.0, np.asarray(scale_exp, dtype=np.int64).reshape(-1))[:, None]
    a = np.abs(xb) / scale
    hi_i = np.clip(np.searchsorted(E2M1, a), 0, len(E2M1) - 1)
    lo_i = np.clip(hi_i - 1, 0, len(E2M1) - 1)
    lo, hi = E2M1[lo_i], E2M1[hi_i]
    take_lo = (a - lo < hi - a) | ((a - lo == hi - a) & (lo_i % 2 == 0))
    mag = np.where(a >= E2M1[-1], E2M1[-1], np.where(take_lo, lo, hi))
    return (np.sign(xb) * mag * scale).reshape(x.shape)


QUANTISERS = {"bf16": lambda s: bf16_round(s), "fp4": lambda s: mxfp4_round(s)}


def quantise_planes(tree: Tree, levels, fmt: str = "bf16") -> Tree:
    """The router's view of a tree whose planes at ``levels`` are stored with s quantised.

    The pages fix no storage precision for the planes (their routing arithmetic is fp32).
    Stated quantisers: "bf16", every element of s_j rounded to the nearest bf16 value;
    "fp4", OCP MX FP4 with one power-of-two scale per 32 elements of each s_j
    (mxfp4_round).  The offsets c_j stay as computed (fp32 storage on the GPU).  The tree
    itself is unchanged: parents and appends keep using the full-precision planes, and only
    routing reads the quantised copy.  Levels not listed keep their full-precision s.
    """
    out = list(tree.levels)
    for lv in levels:
        s, c = tree.levels[lv - 1]
        out[lv - 1] = (QUANTISERS[fmt](s), c)
    return dataclasses.replace(tree, levels=out)


# --------------------------------------------------------------------------- routing
def node_scores(tree: Tree, level: int, nodes: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Router score of each node: the max over its R planes, max_j(sigma q.s_j + c_j).

    [news] "Building the tree": taking the maximum over the reference queries' planes
    approximates the attention any future query gives the block.
    """
    s, c = tree.levels[level - 1]
    q = np.asarray(q, dtype=np.float64)
    sig = 1.0 / math.sqrt(q.shape[0])
    nodes = np.asarray(nodes, dtype=np.int64)
    return np.max(sig * (s[nodes] @ q) + c[nodes], axis=1)


def top_p(frontier: np.ndarray, scores: np.ndarray, p: float) -> dict:
    """Smallest set of frontier nodes whose estimated attention probability reaches p.

    [blog] "Routing through the tree" / [news] "How does top-p routing pick tokens?":
    top-p keeps the smallest group of nodes accounting for a fraction p of the estimated
    attention probability.  Readings: the probabilities are the softmax of the scores
    over the current frontier; "reaching" means cumulative mass >= p; nodes are taken in
    order of decreasing score, equal scores by increasing node id; p >= 1 keeps the whole
    frontier, as does a frontier whose total never reaches p through rounding.
    """
    frontier = np.asarray(frontier, dtype=np.int64)
    scores = np.asarray(scores, dtype=np.float64)
    f = frontier.shape[0]
    if f == 0:
        return dict(order=np.zeros(0, np.int64), pi=np.zeros(0), cum_before=np.zeros(0), k=0,
                    kept=np.zeros(0, np.int64))
    m = np.max(scores)
    e = np.exp(scores - m)
    pi = e / np.sum(e)
    order = np.lexsort((frontier, -scores))
    cum = np.cumsum(pi[order])
    cum_before = np.concatenate([[0.0], cum[:-1]])
    if p >= 1.0:
        k = f
    else:
        hit = np.nonzero(cum >= p)[0]
        k = int(hit[0]) + 1 if hit.size else f
    kept = np.sort(frontier[order[:k]])
    return dict(order=order, pi=pi, cum_before=cum_before, k=k, kept=kept)


def children(tree: Tree, level: int, nodes: np.ndarray) -> np.ndarray:
    """Existing level-(level-1) children of level-``level`` nodes, in id order."""
    b = tree.block
    ch = (np.asarray(nodes, dtype=np.int64)[:, None] * b + np.arange(b)[None, :]).ravel()
    return ch[ch < tree.nodes(level - 1)]


def level_p(p, level: int) -> float:
    """p of the top-p decision at ``level``: a single p for every level, or a schedule
    whose entry level-1 is that level's p.

    [blog] "The narrow path": keeping a fixed fraction at every level compounds over the
    depth, so the threshold would have to change with depth and context; the pages give no
    formula, so a schedule is an input.
    """
    return float(p) if np.ndim(p) == 0 else float(p[level - 1])


def route(tree: Tree, q: np.ndarray, p, keep_sink: bool = True) -> dict:
    """Top-down routing of one query through one tree.

    [blog] "Routing through the tree": score the top level, keep the top-p set, expand
    only the kept nodes' children, repeat down to the raw keys, then attend to the
    selected keys; several branches may stay open.  [news]: the first token is always
    kept as an attention sink.  The level-1 top-p picks blocks and every existing token
    of a kept block is attended; the sink is added after routing (it takes no part in
    the routing mass).  ``p``: one value for every level, or one per level (level_p).
    """
    L = tree.n_levels
    frontier = np.arange(tree.nodes(L), dtype=np.int64)
    per_level = []
    kept = frontier
    for lv in range(L, 0, -1):
        sc = node_scores(tree, lv, frontier, q)
        sel = top_p(frontier, sc, level_p(p, lv))
        per_level.append(dict(level=lv, frontier=frontier, scores=sc, **sel))
        kept = sel["kept"]
        if lv > 1:
            frontier = children(tree, lv, kept)
    b = tree.block
    tok = (kept[:, None] * b + np.arange(b)[None, :]).ravel()
    tok = tok[tok < tree.n_tokens]
    if keep_sink and tree.n_tokens > 0:
        tok = np.union1d(np.array([0], dtype=np.int64), tok)
    return dict(levels=per_level, blocks=kept, tokens=np.sort(tok))


# --------------------------------------------------------------------------- attention
def attend(keys: np.ndarray, values: np.ndarray, q: np.ndarray, tokens: np.ndarray) -> np.ndarray:
    """Ordinary softmax attention of q over the selected raw keys ([blog] "Routing through
    the tree": once the search reaches the raw KV entries, plain attention runs over the
    selected subset)."""
    tokens = np.asarray(tokens, dtype=np.int64)
    k = np.asarray(keys, dtype=np.float64)[tokens]
    v = np.asarray(values, dtype=np.float64)[tokens]
    q = np.asarray(q, dtype=np.float64)
    z = (k @ q) / math.sqrt(q.shape[0])
    w = np.exp(z - np.max(z))
    return (w / np.sum(w)) @ v


def decode(trees: list, values: np.ndarray, q: np.ndarray, p, keep_sink: bool = True,
           return_routes: bool = False):
    """One decode step for all query heads: q [Hq, d], one tree per KV head; query head h
    reads KV head h // (Hq / Hkv) (contiguous groups).  Returns o [Hq, d] (float64)."""
    hq = q.shape[0]
    g = hq // len(trees)
    out = np.zeros((hq, q.shape[1]))
    routes = []
    for h in range(hq):
        t = trees[h // g]
        r = route(t, q[h], p, keep_sink)
        out[h] = attend(t.keys[:t.n_tokens], values[h // g][:t.n_tokens], q[h], r["tokens"])
        routes.append(r)
    return (out, routes) if return_routes else out


def dense_decode(keys: np.ndarray, values: np.ndarray, q: np.ndarray, n_tokens: int) -> np.ndarray:
    """Attention of every query head over all n_tokens keys of its KV head (the dense
    baseline the pages compare against)."""
    hq = q.shape[0]
    g = hq // keys.shape[0]
    all_tok = np.arange(n_tokens)
    return np.stack([attend(keys[h // g], values[h // g], q[h], all_tok) for h in range(hq)])
