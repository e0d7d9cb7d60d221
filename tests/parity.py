"""Comparison helpers for the GPU parity tests (GPU path vs the CPU oracle).

Tolerances (stated once here, used by every GPU test):
  * router scores: |gpu - oracle| <= 1e-4 absolute (fp32 planes and scores);
  * routed sets: identical, except a node whose oracle cumulative probability before it
    lies within 1e-5 of p (its fate flips under rounding of the masses), or whose score is
    within the score tolerance (1e-4) of the boundary node's score (a near tie may swap
    order); end to end, the descendants of such a node are excluded from later levels;
  * outputs: max|o_gpu - o_ref| <= 1e-2 * max|o_ref| (bf16 inputs, fp32 accumulation).

Quantised router planes (bf16, MX FP4): the oracle routes over its planes with s
quantised (oracle ``quantise_planes``) at the levels the router reads planes at.  The GPU
quantises its fp32 s, which lies within S_BAND of the oracle's fp64 s (checked element by
element).  Quantisation is monotone in each element for a fixed block scale, so the GPU's
value lies in [lo, hi]: lo / hi the quantisation of s - S_BAND / s + S_BAND, taken over
every FP4 block scale that an amax within S_BAND can give.  Each node's score tolerance
adds sigma * max_j sum_i |q_i| (hi_ji - lo_ji) (zero where lo = hi, which holds for every
element away from a rounding midpoint or a scale boundary).
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import zha_oracle as zo
from workloads import configs as wc, gen

SCORE_TOL = 1e-4
BAND = 1e-5
OUT_RTOL = 1e-2
S_BAND = 1e-5


def torch_dtype(w: wc.Workload):
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def make_tree(w: wc.Workload, top_p=None, capacity=None):
    from hierarchical_tree_indexed_03_amd import zha
    cfg = zha.make_config(w.head_dim, w.num_kv_heads, w.num_q_heads, w.block, w.levels, w.num_ref,
                          capacity or w.capacity, w.dtype, w.top_p if top_p is None else top_p, w.keep_sink,
                          w.planes)
    return zha.Tree(cfg)


def key_form(w: wc.Workload) -> bool:
    """Level 1 scored from its block's keys and the planes' token weights: bf16 keys, b in
    {2, 4, 8, 16}, and b keys plus R x b fp32 weights take fewer bytes than R fp32 planes
    (the library's rule, which test_abi checks through zha_level1_key_form)."""
    return (w.dtype == "bf16" and w.block in (2, 4, 8, 16)
            and w.block * w.head_dim * 2 + w.num_ref * w.block * 4 < w.num_ref * w.head_dim * 4)


def router_levels(w: wc.Workload) -> list:
    """Levels whose planes the router reads (all but a key-form level 1)."""
    return [lv for lv in range(1, w.levels + 1) if not (lv == 1 and key_form(w))]


def router_trees(w: wc.Workload, trees: list) -> list:
    """The oracle trees as the router sees them: with quantised router planes, s quantised
    at the levels the router reads planes at."""
    if w.planes == "f32":
        return trees
    lv = router_levels(w)
    return [zo.quantise_planes(t, lv, w.planes) for t in trees]


def quant_bounds(fmt: str, s: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """[lo, hi] of the quantised value of every element of s (rows of d) when each element
    may move by up to S_BAND (see the module docstring)."""
    if fmt == "bf16":
        return zo.bf16_round(s - S_BAND), zo.bf16_round(s + S_BAND)
    sb = s.reshape(-1, zo.MX_BLOCK)
    amax = np.max(np.abs(sb), axis=1)
    lo = hi = None
    for a in (np.maximum(amax - S_BAND, 1e-300), amax + S_BAND):
        _, e = np.frexp(a)
        ql = zo.mxfp4_round(sb - S_BAND, e - 3)
        qh = zo.mxfp4_round(sb + S_BAND, e - 3)
        lo = ql if lo is None else np.minimum(lo, ql)
        hi = qh if hi is None else np.maximum(hi, qh)
    tiny = (amax <= S_BAND)[:, None]           # a block within the band of zero
    lo = np.where(tiny, -3 * S_BAND, lo)
    hi = np.where(tiny, 3 * S_BAND, hi)
    return lo.reshape(s.shape), hi.reshape(s.shape)


def flip_allowance(w: wc.Workload, tree, level: int, nodes, q) -> np.ndarray:
    """Extra score tolerance per node for quantised router planes (see the module
    docstring); zero for f32 planes and for a key-form level 1.  ``tree`` is the
    full-precision tree."""
    nodes = np.asarray(nodes, dtype=np.int64)
    if w.planes == "f32" or level not in router_levels(w):
        return np.zeros(len(nodes))
    s = tree.levels[level - 1][0][nodes]
    lo, hi = quant_bounds(w.planes, s)
    return np.max((hi - lo) @ np.abs(np.asarray(q, dtype=np.float64)), axis=1) / np.sqrt(len(q))


E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0])


def decode_fp4(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Values of the GPU's MX FP4 copy (codes [..., d/2] uint8, scales [..., d/32] uint8),
    following the layout zha.h documents."""
    codes = np.asarray(codes, dtype=np.uint8)
    el = np.stack([codes & 0xF, codes >> 4], axis=-1).reshape(*codes.shape[:-1], -1)
    x = np.ldexp(1.0, np.asarray(scales, dtype=np.int64) - 127)
    return E2M1_VALUES[el] * np.repeat(x, zo.MX_BLOCK, axis=-1)


def upload(x: np.ndarray, w: wc.Workload) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch_dtype(w)).cuda()


def host_inputs(w: wc.Workload, n_cap=None):
    K, V = gen.kv_cache(w, n_cap)
    refs = gen.ref_queries(w)
    return K, V, refs


def oracle_trees(w: wc.Workload, K, refs, n_tokens):
    return [zo.build_tree(K[h], refs[h], w.block, w.levels, n_tokens) for h in range(w.num_kv_heads)]


def gpu_kept(trace_level: dict, gi: int) -> np.ndarray:
    nodes = trace_level["nodes"].numpy().astype(np.int64)
    keep = trace_level["keep"].numpy().astype(np.int64) & 0xFFFFFFFF
    return np.sort(nodes[(keep >> gi) & 1 == 1])


def gpu_frontier(trace_level: dict, gi: int) -> np.ndarray:
    nodes = trace_level["nodes"].numpy().astype(np.int64)
    masks = trace_level["masks"].numpy().astype(np.int64) & 0xFFFFFFFF
    return np.sort(nodes[(masks >> gi) & 1 == 1])


def gpu_scores(trace_level: dict, gi: int) -> dict:
    nodes = trace_level["nodes"].numpy().astype(np.int64)
    sc = trace_level["scores"][gi].numpy()
    return dict(zip(nodes.tolist(), sc.tolist()))


def exempt_nodes(rec: dict, p: float, diff: np.ndarray, tol=None) -> tuple[list, list]:
    """Split mismatching nodes into (exempt, failing) per the tolerance rule above.  ``tol``:
    per-frontier-node score tolerance (default SCORE_TOL); a near tie allows the sum of the
    node's and the boundary node's tolerances."""
    frontier = rec["frontier"]
    pos = {int(n): i for i, n in enumerate(frontier)}
    order = rec["order"]
    rank = np.empty(len(order), np.int64)
    rank[order] = np.arange(len(order))
    cum_before = rec["cum_before"]                 # in rank order
    k = rec["k"]
    tol = np.full(len(frontier), SCORE_TOL) if tol is None else np.asarray(tol)
    boundary_score = rec["scores"][order[k - 1]] if k > 0 else np.inf
    boundary_tol = tol[order[k - 1]] if k > 0 else 0.0
    ok, bad = [], []
    for n in diff.tolist():
        i = pos[n]
        cb = cum_before[rank[i]]
        if abs(cb - p) <= BAND or abs(rec["scores"][i] - boundary_score) <= tol[i] + boundary_tol:
            ok.append(n)
        else:
            bad.append((n, float(cb), float(rec["scores"][i] - boundary_score)))
    return ok, bad


def compare_route(route: dict, trace: dict, gi: int, b: int, p, tol_fn=None) -> dict:
    """End-to-end set comparison of one query head.  ``trace[level]`` is the GPU trace of
    that level for the head's KV head (level 0 = kept blocks).  ``p``: one value, or one
    per level (entry level-1).  ``tol_fn(level, frontier)`` gives per-node score tolerances
    (default SCORE_TOL).  Returns a report dict; report["bad"] lists unexplained
    mismatches."""
    excluded = set()
    bad, exempt, n_levels = [], [], len(route["levels"])
    for rec in route["levels"]:
        lv = rec["level"]
        tl = trace[lv]
        f_o = set(rec["frontier"].tolist()) - excluded
        f_g = set(gpu_frontier(tl, gi).tolist()) - excluded
        if f_o != f_g:
            bad.append(("frontier", lv, sorted(f_o ^ f_g)[:10]))
            break
        k_o = set(rec["kept"].tolist()) - excluded
        k_g = set(gpu_kept(tl, gi).tolist()) - excluded
        diff = np.array(sorted(k_o ^ k_g), dtype=np.int64)
        tol = None if tol_fn is None else tol_fn(lv, rec["frontier"])
        ok, nb = exempt_nodes(rec, p if np.ndim(p) == 0 else p[lv - 1], diff, tol)
        exempt += [(lv, n) for n in ok]
        bad += [("kept", lv) + x for x in nb]
        if lv == 1:
            # the gathered blocks are level-1 nodes: an exempt one is excluded itself
            excluded = excluded | set(ok)
            break
        nxt = set()
        for n in excluded | set(ok):
            nxt.update(range(n * b, n * b + b))
        excluded = nxt
    # gathered blocks (level 0 of the trace) = kept level-1 blocks
    k_o = set(route["blocks"].tolist()) - excluded
    k_g = set(gpu_frontier(trace[0], gi).tolist()) - excluded
    if k_o != k_g:
        bad.append(("blocks", 0, sorted(k_o ^ k_g)[:10]))
    return dict(bad=bad, exempt=exempt)


def gpu_tokens(trace0: dict, gi: int, b: int, n_tokens: int, keep_sink=True) -> np.ndarray:
    blocks = gpu_frontier(trace0, gi)
    tok = (blocks[:, None] * b + np.arange(b)[None, :]).ravel()
    tok = tok[tok < n_tokens]
    if keep_sink:
        tok = np.union1d([0], tok)
    return np.sort(tok)


def out_err(o_gpu: np.ndarray, o_ref: np.ndarray) -> float:
    return float(np.max(np.abs(o_gpu - o_ref)) / max(1e-30, np.max(np.abs(o_ref))))


def fit_flip_allowance(keys, refs, block, levels, n_tokens, queries, tol=2 * SCORE_TOL) -> np.ndarray:
    """Per-element allowance [R, d] for the fitting gradient: a (query, node) whose two best
    planes lie within `tol` of each other may take either as its arg-max on the GPU, which
    moves that pair's contribution g * sigma^2 C_p (q - r_p) between the two planes; the
    allowance adds the absolute contribution of both (divided by the number of queries, as
    the gradient is a mean)."""
    import math
    keys = np.asarray(keys, dtype=np.float64)
    refs = np.asarray(refs, dtype=np.float64)
    queries = np.asarray(queries, dtype=np.float64)
    d = keys.shape[1]
    sig = 1.0 / math.sqrt(d)
    tree = zo.build_tree(keys, refs, block, levels, n_tokens)
    allow = np.zeros_like(refs)
    if refs.shape[0] < 2:
        return allow
    for lv in range(1, levels + 1):
        s, c = tree.levels[lv - 1]
        span = block ** lv
        for q in queries:
            f = sig * (s @ q) + c
            top = np.sort(f, axis=1)
            near = np.nonzero(top[:, -1] - top[:, -2] < tol)[0]
            if near.size == 0:
                continue
            logm = zo.node_log_mass(keys, q, block, lv, n_tokens)
            logpi, _ = zo.router_log_probs(tree, lv, q)
            g = np.exp(logpi) - np.exp(logm)
            for n in near:
                toks = keys[n * span:min((n + 1) * span, n_tokens)]
                for p in np.argsort(f[n])[-2:]:
                    z = sig * toks @ refs[p]
                    w = np.exp(z - np.max(z))
                    w /= w.sum()
                    diff = toks - s[n, p]
                    allow[p] += np.abs(g[n] * sig * sig * ((w * (diff @ (q - refs[p]))) @ diff))
    return allow / len(queries)
