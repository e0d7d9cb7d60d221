"""Comparison helpers for the GPU parity tests (GPU path vs the CPU oracle).

Tolerances (stated once here, used by every GPU test):
  * router scores: |gpu - oracle| <= 1e-4 absolute (fp32 planes and scores);
  * routed sets: at every level the GPU's kept set must be the oracle's top-p of the same
    frontier under the oracle's scores.  Two departures are explained, nothing else:
      - a near-tie swap: an oracle-kept node the GPU dropped, paired one to one with a node
        the GPU kept instead, whose oracle scores differ by at most the two nodes' score
        tolerances and which the GPU's own scores rank ahead of the dropped one (pairs are
        formed first, so that a swap whose added node happens to lie in the band does not
        leave its dropped node unexplained);
      - the mass band: a node whose oracle cumulative probability before it (in oracle rank
        order) lies within 1e-5 of p may be kept or dropped (the rounding of the masses may
        flip it); this is the only way the kept count may differ.
    End to end the comparison walks the GPU's own frontiers (each the existing children of
    the GPU's kept nodes one level up), so a legitimate departure never masks a later
    level; the number of departures is reported per test and bounded by stated rates;
  * outputs: max|o_gpu - o_ref| <= 1e-2 * max|o_ref| (bf16 inputs, fp32 accumulation),
    against attention over the GPU's gathered set always, and against the oracle's own
    decode whenever the GPU took the oracle's route (no departure at any level).

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


def router_levels(w: wc.Workload, keys: bool = False) -> list:
    """Levels whose planes the router reads (all but a key-form level 1; none when every
    level is scored from the keys, ``keys``)."""
    if keys:
        return []
    return [lv for lv in range(1, w.levels + 1) if not (lv == 1 and key_form(w))]


def router_trees(w: wc.Workload, trees: list, keys: bool = False) -> list:
    """The oracle trees as the router sees them: with quantised router planes, s quantised
    at the levels the router reads planes at (none when every level is scored from the
    keys, ``keys``)."""
    if w.planes == "f32" or keys:
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


def flip_allowance(w: wc.Workload, tree, level: int, nodes, q, keys: bool = False) -> np.ndarray:
    """Extra score tolerance per node for quantised router planes (see the module
    docstring); zero for f32 planes, for a key-form level 1 and for every level when all
    are scored from the keys (``keys``).  ``tree`` is the full-precision tree."""
    nodes = np.asarray(nodes, dtype=np.int64)
    if w.planes == "f32" or level not in router_levels(w, keys):
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


def gpu_scores_on(trace_level: dict, gi: int, nodes) -> np.ndarray:
    """GPU scores of head gi for the given nodes (each must be in the trace's list)."""
    tn = trace_level["nodes"].numpy().astype(np.int64)
    nodes = np.asarray(nodes, dtype=np.int64)
    pos = np.searchsorted(tn, nodes)
    assert np.all(pos < len(tn)) and np.array_equal(tn[np.minimum(pos, len(tn) - 1)], nodes), "node not in trace"
    return trace_level["scores"][gi].numpy().astype(np.float64)[pos]


def _rank_order(frontier: np.ndarray, scores: np.ndarray) -> np.ndarray:
    """Position of every frontier node in the top-p rank order (score descending, equal
    scores by node id ascending)."""
    order = np.lexsort((frontier, -np.asarray(scores, dtype=np.float64)))
    rank = np.empty(len(order), np.int64)
    rank[order] = np.arange(len(order))
    return rank


def check_selection(frontier, s_ref, s_gpu, kept_gpu, p: float, tol=None) -> dict:
    """One query head's top-p decision at one level, on a given frontier.

    ``s_ref``: the oracle's scores of the frontier nodes; ``s_gpu``: the GPU's; ``kept_gpu``:
    the nodes the GPU kept.  The expected set is the oracle's top_p of (frontier, s_ref).
    A difference is explained only by
      * the mass band: a node whose oracle cumulative probability before it lies within
        BAND of p (the rounding of the masses may flip it); this is the only way the kept
        count may differ;
      * a near-tie swap: an oracle-kept node the GPU dropped, paired one to one with a node
        the GPU kept instead, whose oracle scores differ by at most the two nodes' score
        tolerances and which the GPU's own scores rank ahead of it.
    Anything else is returned in ``bad``.  ``tol``: per-frontier-node score tolerance
    (default SCORE_TOL)."""
    frontier = np.asarray(frontier, dtype=np.int64)
    s_ref = np.asarray(s_ref, dtype=np.float64)
    s_gpu = np.asarray(s_gpu, dtype=np.float64)
    tol = np.full(len(frontier), SCORE_TOL) if tol is None else np.asarray(tol, dtype=np.float64)
    rec = zo.top_p(frontier, s_ref, p)
    out = dict(bad=[], band=[], swap=[], k=rec["k"])
    pos = {int(n): i for i, n in enumerate(frontier.tolist())}
    kept_gpu = [int(n) for n in np.asarray(kept_gpu).tolist()]
    stray = [n for n in kept_gpu if n not in pos]
    if stray:
        out["bad"].append(("outside frontier", stray[:5]))
        return out
    if len(frontier) == 0:
        return out
    rank = _rank_order(frontier, s_ref)
    grank = _rank_order(frontier, s_gpu)
    cb = rec["cum_before"]
    k_o = set(rec["kept"].tolist())
    k_g = set(kept_gpu)
    in_band = lambda n: abs(cb[rank[pos[n]]] - p) <= BAND
    dropped = sorted((n for n in k_o - k_g), key=lambda n: rank[pos[n]])
    added = sorted((n for n in k_g - k_o), key=lambda n: rank[pos[n]])
    # near-tie swaps first (a swap's two nodes may also lie in the band; pairing them keeps
    # the band for a node the cut itself moved), then the band
    used, paired = set(), set()
    for d in dropped:
        i = pos[d]
        for a in added:
            j = pos[a]
            if a in used:
                continue
            if abs(s_ref[i] - s_ref[j]) <= tol[i] + tol[j] and grank[j] < grank[i]:
                used.add(a)
                paired.add(d)
                out["swap"].append((d, a))
                break
    dropped = [n for n in dropped if n not in paired]
    added = [n for n in added if n not in used]
    out["band"] = [n for n in dropped + added if in_band(n)]
    bnd = s_ref[rec["order"][rec["k"] - 1]] if rec["k"] > 0 else np.inf
    for n in dropped:
        if not in_band(n):
            i = pos[n]
            out["bad"].append(("dropped", n, float(cb[rank[i]]), float(s_ref[i] - bnd)))
    for n in added:
        if not in_band(n):
            j = pos[n]
            out["bad"].append(("added", n, float(cb[rank[j]]), float(s_ref[j] - bnd)))
    return out


def new_report() -> dict:
    return dict(bad=[], band=0, swap=0, selections=0, same=True)


def compare_route(tree, q, trace: dict, gi: int, p, tol_fn=None) -> dict:
    """End-to-end check of one query head's routing, walking the GPU's own frontiers.

    ``tree``: the oracle tree the router reads (for quantised router planes, the oracle's
    quantised copy); ``trace[level]``: the GPU trace of the head's KV head (level 0 = the
    gathered blocks).  At every level from the top:
      * the GPU frontier must be every node (top level) or exactly the existing children
        of the nodes the GPU kept one level up;
      * the GPU score of every frontier node must be within the score tolerance of the
        oracle's score of that node (``tol_fn(level, frontier)``, default SCORE_TOL);
      * the GPU kept set must be the oracle's top-p of that frontier under the oracle's
        scores (check_selection: the mass band and verified near-tie swaps only).
    The gathered blocks must be the kept level-1 nodes.  ``same`` is True when no exemption
    was used, i.e. the GPU took the oracle's own route, whose output the caller may then
    compare with the oracle's.  ``p``: one value, or one per level (entry level-1)."""
    rep = new_report()
    L = tree.n_levels
    prev = None
    for lv in range(L, 0, -1):
        fr = gpu_frontier(trace[lv], gi)
        want = np.arange(tree.nodes(lv), dtype=np.int64) if prev is None else zo.children(tree, lv + 1, prev)
        if not np.array_equal(fr, np.sort(want)):
            rep["bad"].append(("frontier", lv, sorted(set(fr.tolist()) ^ set(want.tolist()))[:10]))
            return rep
        s_ref = zo.node_scores(tree, lv, fr, q)
        s_gpu = gpu_scores_on(trace[lv], gi, fr)
        tol = np.full(len(fr), SCORE_TOL) if tol_fn is None else np.asarray(tol_fn(lv, fr), dtype=np.float64)
        over = np.abs(s_gpu - s_ref) - tol
        if len(fr) and np.max(over) > 0:
            i = int(np.argmax(over))
            rep["bad"].append(("score", lv, int(fr[i]), float(s_gpu[i]), float(s_ref[i])))
            return rep
        sel = check_selection(fr, s_ref, s_gpu, gpu_kept(trace[lv], gi), zo.level_p(p, lv), tol)
        rep["selections"] += 1
        rep["band"] += len(sel["band"])
        rep["swap"] += len(sel["swap"])
        if sel["bad"]:
            rep["bad"] += [("kept", lv) + tuple(x) for x in sel["bad"]]
            return rep
        prev = gpu_kept(trace[lv], gi)
    blocks = gpu_frontier(trace[0], gi)
    if not np.array_equal(blocks, prev):
        rep["bad"].append(("blocks", sorted(set(blocks.tolist()) ^ set(prev.tolist()))[:10]))
    rep["same"] = rep["band"] == 0 and rep["swap"] == 0
    return rep


def union_frontiers(routes: list, li: int, hkv: int, g: int) -> list:
    """The group unions of the oracle routes' frontiers at entry li of route["levels"]:
    per KV head (node ids ascending, head masks)."""
    fronts = []
    for kv in range(hkv):
        fr = {}
        for gi in range(g):
            for n in routes[kv * g + gi]["levels"][li]["frontier"].tolist():
                fr[n] = fr.get(n, 0) | (1 << gi)
        nodes = np.array(sorted(fr), dtype=np.int64)
        fronts.append((nodes, np.array([fr[n] for n in nodes.tolist()], dtype=np.int64)))
    return fronts


def teacher_forced(t, trees: list, q: np.ndarray, qd, p, keep_sink: bool, path: int = 0,
                   tol_fn=None) -> dict:
    """Teacher-forced routing through the C ABI: at every level the GPU routes the oracle's
    own frontier (zha_debug_route_level; path 0 = the kernels zha_decode runs at that level,
    1 = the list path), and its scores and kept sets are checked with check_selection.
    ``trees``: the router's oracle trees per KV head; ``tol_fn(kv, q_head)`` returns a
    per-level tolerance function as compare_route takes.  Returns a report (bad, band,
    swap, selections, max score error)."""
    hkv = len(trees)
    hq = q.shape[0]
    g = hq // hkv
    L = trees[0].n_levels
    routes = [zo.route(trees[h // g], q[h], p, keep_sink) for h in range(hq)]
    rep = new_report()
    rep["max_err"] = 0.0
    for li in range(L):
        lv = L - li
        tr = t.route_level(lv, qd, union_frontiers(routes, li, hkv, g), path)
        for h in range(hq):
            kv, gi = divmod(h, g)
            rec = routes[h]["levels"][li]
            fr = rec["frontier"]
            s_gpu = gpu_scores_on(tr[kv], gi, fr)
            tol = (np.full(len(fr), SCORE_TOL) if tol_fn is None
                   else np.asarray(tol_fn(kv, q[h])(lv, fr), dtype=np.float64))
            err = np.abs(s_gpu - rec["scores"])
            rep["max_err"] = max(rep["max_err"], float(np.max(err)) if len(fr) else 0.0)
            if len(fr) and np.any(err > tol):
                i = int(np.argmax(err - tol))
                rep["bad"].append(("score", lv, h, int(fr[i]), float(s_gpu[i]), float(rec["scores"][i])))
                continue
            sel = check_selection(fr, rec["scores"], s_gpu, gpu_kept(tr[kv], gi), zo.level_p(p, lv), tol)
            rep["selections"] += 1
            rep["band"] += len(sel["band"])
            rep["swap"] += len(sel["swap"])
            rep["bad"] += [("kept", lv, h) + tuple(x) for x in sel["bad"]]
    return rep


# Exemptions expected at most: the masses are fixed-point on the GPU (about 1e-7 relative to
# the oracle's), so a mass-band flip needs a boundary within ~1e-7 of p although the band is
# 1e-5 wide; a swap needs two boundary-adjacent scores closer than the fp32 score error
# (about 1e-6).  Both are rare on these inputs: over the whole GPU suite (about 15,000 level
# selections) one band flip and no swap, apart from inputs built to sit exactly on p.
MAX_BAND_RATE = 0.02
MAX_SWAP_RATE = 0.02


def merge_reports(reps) -> dict:
    tot = new_report()
    for r in reps:
        tot["bad"] += r["bad"]
        for k in ("band", "swap", "selections"):
            tot[k] += r.get(k, 0)
        tot["same"] = tot["same"] and r.get("same", True)
    return tot


def assert_exemption_rates(label: str, reps, band_rate: float = MAX_BAND_RATE) -> dict:
    """Prints the exemption counts of a test's level selections and fails when they exceed
    the stated rates (band_rate, MAX_SWAP_RATE of the selections, at least 2 each).  Inputs
    built to put the boundary exactly on p (equal masses) pass a band_rate of 1."""
    tot = merge_reports(reps) if isinstance(reps, (list, tuple)) else reps
    sel = tot["selections"]
    print(f"[exemptions] {label}: {sel} level selections, {tot['band']} mass-band, {tot['swap']} near-tie swaps")
    assert tot["band"] <= max(2, band_rate * sel), f"{label}: {tot['band']} mass-band exemptions in {sel}"
    assert tot["swap"] <= max(2, MAX_SWAP_RATE * sel), f"{label}: {tot['swap']} near-tie swaps in {sel}"
    return tot


def check_decode(trees: list, K, V, q: np.ndarray, o: np.ndarray, traces: dict, p, keep_sink: bool, n: int,
                 tol_fn=None, label: str = "") -> list:
    """One decode step of every query head against the oracle: compare_route on the GPU's
    trace (``traces[level][kv]``), attention over the GPU's gathered tokens, and the
    oracle's own decode output whenever the GPU took the oracle's route.  ``trees``: the
    router's oracle trees per KV head (their keys are the caches); ``K``, ``V``: host caches
    [Hkv, >= n, d]; ``tol_fn(kv, q_head)`` -> per-level tolerance as compare_route takes.
    Returns the per-head reports."""
    hkv = len(trees)
    hq = q.shape[0]
    g = hq // hkv
    b = trees[0].block
    o_ref = zo.decode(trees, V, q, p, keep_sink)
    reps = []
    for h in range(hq):
        kv, gi = divmod(h, g)
        tr = {lv: traces[lv][kv] for lv in traces}
        rep = compare_route(trees[kv], q[h], tr, gi, p, None if tol_fn is None else tol_fn(kv, q[h]))
        assert not rep["bad"], f"{label} head {h}: {rep['bad'][:5]}"
        toks = gpu_tokens(tr[0], gi, b, n, keep_sink)
        e1 = out_err(o[h], zo.attend(K[kv][:n], V[kv][:n], q[h], toks))
        assert e1 <= OUT_RTOL, f"{label} head {h}: attention over the GPU's set, error {e1:.3e}"
        if rep["same"]:
            e2 = out_err(o[h], o_ref[h])
            assert e2 <= OUT_RTOL, f"{label} head {h}: output error {e2:.3e} against the oracle's decode"
        reps.append(rep)
    return reps


def kept_from_bits(words, n: int) -> np.ndarray:
    """Node ids set in a kept bitmap (uint32 words, bit e % 32 of word e // 32 = node e)."""
    w = np.ascontiguousarray(np.asarray(words).astype(np.int64) & 0xFFFFFFFF, dtype="<u4")
    bits = np.unpackbits(w.view(np.uint8), bitorder="little")
    return np.nonzero(bits[:n])[0].astype(np.int64)


def compare_prefill_pair(tree, q, scores: dict, kept: dict, p) -> tuple:
    """One (query, head) pair of a batched prefill against ``tree``, the oracle tree of the
    tokens up to and including the query's own.  ``scores[lv]``: the GPU's score row of the
    pair over every node of the sub-batch's tree at level lv; ``kept[lv]``: the node ids the
    GPU kept.  At every level from the top:
      * every node of the pair's tree scores within SCORE_TOL of the oracle's score (the
        rightmost one is the pair's own version of that node), every node right of it
        scores -inf;
      * the GPU's kept set is the oracle's top-p of the GPU's frontier (every node at the
        top, else the children of the GPU's kept nodes one level up), by check_selection.
    Returns (report, kept level-1 blocks)."""
    rep = new_report()
    prev = None
    for lv in range(tree.n_levels, 0, -1):
        n = tree.nodes(lv)
        row = np.asarray(scores[lv], dtype=np.float64)
        if len(row) < n or np.any(row[n:] != -np.inf):
            rep["bad"].append(("tail", lv, n, len(row)))
            return rep, None
        s_ref = zo.node_scores(tree, lv, np.arange(n, dtype=np.int64), q)
        err = np.abs(row[:n] - s_ref)
        if n and np.max(err) > SCORE_TOL:
            i = int(np.argmax(err))
            rep["bad"].append(("score", lv, i, float(row[i]), float(s_ref[i])))
            return rep, None
        fr = np.arange(n, dtype=np.int64) if prev is None else zo.children(tree, lv + 1, prev)
        sel = check_selection(fr, s_ref[fr], row[fr], kept[lv], zo.level_p(p, lv))
        rep["selections"] += 1
        rep["band"] += len(sel["band"])
        rep["swap"] += len(sel["swap"])
        if sel["bad"]:
            rep["bad"] += [("kept", lv) + tuple(x) for x in sel["bad"]]
            return rep, None
        prev = np.sort(np.asarray(kept[lv], dtype=np.int64))
    rep["same"] = rep["band"] == 0 and rep["swap"] == 0
    return rep, prev


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
