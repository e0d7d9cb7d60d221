"""The GPU-vs-oracle set comparator (tests/parity.py) on planted decisions, on the CPU.

A comparator that accepts a wrong cut proves nothing, so each way a top-p decision can go
wrong is planted into an otherwise exact decision and must be reported:
  * one node too few (keep k-1) or too many (keep k+1): allowed only where the oracle's
    cumulative probability before the node lies within 1e-5 of p (the mass band);
  * a swap of the boundary node for the next one: allowed only when their oracle scores
    are within the two score tolerances AND the GPU's own scores rank the added node first;
  * a dropped node far from the boundary, a node outside the frontier.
The end-to-end walk (compare_route) must also catch a wrong expansion, a score beyond the
tolerance and a gather list that is not the kept level-1 set.
"""
from __future__ import annotations

import numpy as np
import torch

import parity as P
from oracle import zha_oracle as zo


def frontier_case(rng, n=None, spread=None):
    n = int(rng.integers(1_000, 30_000)) if n is None else n
    spread = float(rng.uniform(0.3, 3.0)) if spread is None else spread
    frontier = np.sort(rng.choice(4 * n, n, replace=False)).astype(np.int64)
    scores = rng.standard_normal(n) * spread
    return frontier, scores


def ranked(frontier, scores):
    return frontier[np.lexsort((frontier, -scores))]


def test_exact_decision_passes():
    rng = np.random.default_rng(0)
    for _ in range(50):
        fr, s = frontier_case(rng)
        p = float(rng.uniform(0.3, 0.99))
        rec = zo.top_p(fr, s, p)
        out = P.check_selection(fr, s, s.astype(np.float32), rec["kept"], p)
        assert not out["bad"] and not out["band"] and not out["swap"]


def test_keep_one_fewer_or_more_is_caught():
    """keep k-1 and keep k+1: reported unless the boundary lies in the 1e-5 mass band."""
    rng = np.random.default_rng(1)
    flagged = {"fewer": 0, "more": 0}
    trials = 300
    for _ in range(trials):
        fr, s = frontier_case(rng)
        p = float(rng.uniform(0.3, 0.99))
        rec = zo.top_p(fr, s, p)
        order = ranked(fr, s)
        k = rec["k"]
        cb = rec["cum_before"]
        if k >= 2:
            fewer = np.sort(order[:k - 1])
            out = P.check_selection(fr, s, s, fewer, p)
            in_band = abs(cb[k - 1] - p) <= P.BAND
            assert bool(out["bad"]) == (not in_band)
            flagged["fewer"] += bool(out["bad"])
        if k < len(fr):
            more = np.sort(order[:k + 1])
            out = P.check_selection(fr, s, s, more, p)
            in_band = abs(cb[k] - p) <= P.BAND
            assert bool(out["bad"]) == (not in_band)
            flagged["more"] += bool(out["bad"])
    # the band holds the boundary with probability about 1e-5 / (the boundary node's
    # probability), up to a third on 30K-node frontiers of small spread: most cuts are caught
    assert flagged["fewer"] >= 0.8 * trials and flagged["more"] >= 0.8 * trials, flagged


def test_swaps():
    """The boundary node exchanged for the next-ranked one."""
    rng = np.random.default_rng(2)
    for trial in range(100):
        fr, s = frontier_case(rng, n=5_000)
        p = float(rng.uniform(0.5, 0.95))
        rec = zo.top_p(fr, s, p)
        order_idx = np.lexsort((fr, -s))
        k = rec["k"]
        if k >= len(fr) or k < 2:
            continue
        i, j = order_idx[k - 1], order_idx[k]          # boundary node, first dropped node
        if abs(rec["cum_before"][k - 1] - p) <= P.BAND or abs(rec["cum_before"][k] - p) <= P.BAND:
            continue
        kept_swapped = np.sort(np.concatenate([fr[order_idx[:k - 1]], [fr[j]]]))
        # near tie: put node j within 5e-5 below node i on the oracle side, GPU ranks j first
        s2 = s.copy()
        s2[j] = s2[i] - 5e-5
        rec2 = zo.top_p(fr, s2, p)
        if rec2["k"] != k or not np.array_equal(rec2["kept"], rec["kept"]):
            continue
        if abs(rec2["cum_before"][k - 1] - p) <= P.BAND or abs(rec2["cum_before"][k] - p) <= P.BAND:
            continue
        g = s2.copy()
        g[j] = s2[i] + 1e-6                               # the GPU's scores reverse the pair
        out = P.check_selection(fr, s2, g, kept_swapped, p)
        assert not out["bad"] and len(out["swap"]) == 1, out
        # the same swap without the GPU's scores reversing the pair: reported
        out = P.check_selection(fr, s2, s2, kept_swapped, p)
        assert out["bad"], "swap accepted although the GPU's own scores keep the order"
        # a swap across a gap wider than the tolerances: reported
        s3 = s.copy()
        s3[j] = s3[i] - 5e-3
        rec3 = zo.top_p(fr, s3, p)
        if rec3["k"] == k and np.array_equal(rec3["kept"], rec["kept"]):
            g3 = s3.copy()
            g3[j] = s3[i] + 1e-6
            out = P.check_selection(fr, s3, g3, kept_swapped, p)
            assert out["bad"], "swap across 5e-3 accepted"


def test_far_node_and_stray_node_caught():
    rng = np.random.default_rng(3)
    fr, s = frontier_case(rng, n=2_000)
    p = 0.9
    rec = zo.top_p(fr, s, p)
    order = ranked(fr, s)
    out = P.check_selection(fr, s, s, np.sort(order[1:rec["k"]]), p)   # top node dropped
    assert out["bad"]
    stray = np.sort(np.concatenate([rec["kept"], [4 * len(fr) + 7]]))
    out = P.check_selection(fr, s, s, stray, p)
    assert out["bad"]


def test_band_exemption_counted():
    """A boundary placed inside the band: the flip is accepted and counted."""
    fr = np.arange(4, dtype=np.int64)
    s = np.log(np.array([0.5, 0.3, 0.2 - 4e-6, 4e-6]))   # cumulative 0.5, 0.8, 1-4e-6
    p = 0.8 + 3e-6
    rec = zo.top_p(fr, s, p)
    assert rec["k"] == 3
    out = P.check_selection(fr, s, s, np.array([0, 1]), p)   # the GPU stopped at 0.8
    assert not out["bad"] and out["band"] == [2]


def _trace_of_route(route, tree, q, n_top):
    """A GPU-like trace of one head (group slot 0) that follows the oracle route exactly."""
    tr = {}
    for rec in route["levels"]:
        fr = rec["frontier"]
        sc = torch.zeros(8, len(fr), dtype=torch.float32)
        sc[0] = torch.from_numpy(rec["scores"].astype(np.float32))
        keep = np.isin(fr, rec["kept"]).astype(np.int32)
        tr[rec["level"]] = dict(nodes=torch.from_numpy(fr.astype(np.int32)),
                                masks=torch.ones(len(fr), dtype=torch.int32),
                                scores=sc, keep=torch.from_numpy(keep))
    bl = route["blocks"]
    tr[0] = dict(nodes=torch.from_numpy(bl.astype(np.int32)), masks=torch.ones(len(bl), dtype=torch.int32),
                 scores=None, keep=None)
    return tr


def test_compare_route_walk():
    rng = np.random.default_rng(4)
    n, d = 3_000, 16
    keys = rng.standard_normal((n, d))
    refs = rng.standard_normal((3, d))
    tree = zo.build_tree(keys, refs, 4, 4, n)
    q = keys[rng.choice(n, 3, replace=False)].sum(0)
    q = 4 * np.sqrt(d) * q / np.linalg.norm(q)
    p = 0.9
    route = zo.route(tree, q, p)
    tr = _trace_of_route(route, tree, q, tree.nodes(4))
    rep = P.compare_route(tree, q, tr, 0, p)
    assert not rep["bad"] and rep["same"] and rep["selections"] == 4
    # a score beyond the tolerance
    bad = {lv: dict(v) for lv, v in tr.items()}
    sc = bad[2]["scores"].clone()
    sc[0, 0] += 3e-4
    bad[2]["scores"] = sc
    assert P.compare_route(tree, q, bad, 0, p)["bad"][0][0] == "score"
    # a wrong expansion: one child missing from the level-2 frontier
    bad = {lv: dict(v) for lv, v in tr.items()}
    keep = bad[2]["nodes"].numpy()
    bad[2] = {k: (v[1:] if v is not None and k != "scores" else (v[:, 1:] if v is not None else v))
              for k, v in bad[2].items()}
    assert P.compare_route(tree, q, bad, 0, p)["bad"][0][0] == "frontier"
    # a gather list that is not the kept level-1 set
    bad = {lv: dict(v) for lv, v in tr.items()}
    bad[0] = dict(tr[0])
    bad[0]["nodes"] = tr[0]["nodes"][1:]
    bad[0]["masks"] = tr[0]["masks"][1:]
    assert P.compare_route(tree, q, bad, 0, p)["bad"][0][0] == "blocks"
    # one kept node too few at level 1 (outside the band)
    rec1 = route["levels"][-1]
    cb = rec1["cum_before"][rec1["k"] - 1]
    if abs(cb - p) > P.BAND and rec1["k"] > 1:
        order = ranked(rec1["frontier"], rec1["scores"])
        bad = {lv: dict(v) for lv, v in tr.items()}
        keep = np.isin(rec1["frontier"], order[:rec1["k"] - 1]).astype(np.int32)
        bad[1]["keep"] = torch.from_numpy(keep)
        bad[0]["nodes"] = torch.from_numpy(np.sort(order[:rec1["k"] - 1]).astype(np.int32))
        bad[0]["masks"] = torch.ones(rec1["k"] - 1, dtype=torch.int32)
        assert P.compare_route(tree, q, bad, 0, p)["bad"][0][0] == "kept"


def test_swap_whose_mate_lies_in_the_band():
    """A near-tie pair reversed by the GPU's scores where the added node's oracle cumulative
    probability lies in the band and the dropped node's does not: one swap, nothing bad
    (the band must not take the swap's mate and leave the dropped node unexplained)."""
    p = 0.95
    big = [0.5, 0.3, p - 1.6e-5 - 0.8]                 # three nodes 1.6e-5 short of p
    pa = 2.32e-5                                       # node A: the oracle's boundary node
    filler = np.full(3000, (1.0 - sum(big) - 2 * pa) / 3000)   # each smaller than A and B
    pi = np.concatenate([big, [pa, pa], filler])
    s = np.log(pi)
    s[4] = s[3] - 2e-7                                 # node B, a near tie just after A
    fr = np.arange(len(pi), dtype=np.int64)
    rec = zo.top_p(fr, s, p)
    cb = rec["cum_before"][np.argsort(rec["order"])]
    assert list(rec["kept"]) == [0, 1, 2, 3]
    assert abs(cb[3] - p) > P.BAND and abs(cb[4] - p) <= P.BAND
    g = s.copy()
    g[3], g[4] = s[4], s[3]                            # the GPU ranks B before A
    kept_g = zo.top_p(fr, g, p)["kept"]
    assert list(kept_g) == [0, 1, 2, 4]
    out = P.check_selection(fr, s, g, kept_g, p)
    assert not out["bad"] and out["swap"] == [(3, 4)], out
