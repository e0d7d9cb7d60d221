"""The 16M-token ultra workload against the oracle's full routed sets (CPU).

The GPU side is a saved trace of one decode step (tests/data/make_ultra_trace.py, run
through the C ABI in the launch configuration bench.py times): for the 8 query heads of KV
head 0, the kept node ids of every level, the GPU scores of the frontier nodes near each
boundary, the gathered blocks, the queries and the outputs.  Here the oracle rebuilds that
KV head's whole tree over the 16,777,217 seeded tokens (level 1 chunk by chunk, every
level above from the one below, in float64) and, for every head and level, walks the
GPU's own frontier (the children of the GPU's kept nodes one level up): the GPU's kept set
must be the oracle's top-p of that frontier under the oracle's scores, up to the 1e-5 mass
band and near-tie swaps that the GPU's saved scores reverse (tests/parity.py).  The saved
GPU scores must match the oracle's within 1e-4, the gathered blocks must be the kept
level-1 nodes, the output must match attention over the gathered tokens, and where no
exemption was used the kept sets must equal the oracle's own route at every level.
"""
from __future__ import annotations

import os

import numpy as np
import pytest

import parity as P
from oracle import zha_oracle as zo
from workloads import configs as wc, gen

DATA = os.path.join(os.path.dirname(os.path.abspath(__file__)), "data", "ultra_16m_kv0_trace.npz")


def build_kv0(w, n):
    """Oracle tree of KV head 0 over tokens [0, n): level 1 per 2^20-token chunk (a block never
    straddles a chunk), levels above from the level below; the keys kept as bf16 bit
    patterns for the attention."""
    refs = gen.ref_queries(w)[0].astype(np.float64)
    kbits = np.empty((n, w.head_dim), np.uint16)
    s1, c1 = [], []
    for lo in range(0, n, gen.CHUNK):
        hi = min(n, lo + gen.CHUNK)
        rows = gen.token_rows(w, gen.STREAM_K, 0, lo, hi)
        kbits[lo:hi] = (rows.view(np.uint32) >> 16).astype(np.uint16)
        s, c = zo.level1_planes(rows.astype(np.float64), refs, w.block)
        s1.append(s)
        c1.append(c)
    levels = [(np.concatenate(s1), np.concatenate(c1))]
    del s1, c1
    for _ in range(2, w.levels + 1):
        levels.append(zo.parent_planes(levels[-1][0], levels[-1][1], refs, w.block))
    tree = zo.Tree(keys=np.zeros((0, w.head_dim)), refs=refs, block=w.block, n_levels=w.levels, n_tokens=n,
                   levels=levels)
    return tree, kbits


def rows_of(bits, idx):
    return gen.bf16_to_f32(bits[idx]).astype(np.float64)


@pytest.fixture(scope="module")
def case():
    if not os.path.exists(DATA):
        pytest.fail(f"{DATA} is missing (written by tests/data/make_ultra_trace.py on a GPU)")
    rec = dict(np.load(DATA))
    w = wc.ULTRA.with_(steps=1)
    n = int(rec["n_tokens"])
    assert n == w.n_tokens + 1
    tree, kbits = build_kv0(w, n)
    return w, n, rec, tree, kbits


def test_queries_regenerate(case):
    """The saved queries are the seeded planted queries of the step (same bits)."""
    w, n, rec, tree, kbits = case
    for gi in range(w.group):
        q, _ = gen.planted_query(w, 0, gi, n, lambda kv, idx: gen.bf16_to_f32(kbits[idx]))
        assert np.array_equal(q, rec["q"][gi])


def test_routed_sets_and_outputs(case):
    w, n, rec, tree, kbits = case
    p, b, L = w.top_p, w.block, w.levels
    reps, tokens = [], {}
    for gi in range(w.group):
        q = rec["q"][gi].astype(np.float64)
        rep = P.new_report()
        prev = None
        for lv in range(L, 0, -1):
            fr = np.arange(tree.nodes(lv), dtype=np.int64) if prev is None else zo.children(tree, lv + 1, prev)
            s_ref = zo.node_scores(tree, lv, fr, q)
            near = rec[f"near_l{lv}_g{gi}"].astype(np.int64)
            pos = np.searchsorted(fr, near)
            assert np.all(pos < len(fr)) and np.array_equal(fr[np.minimum(pos, len(fr) - 1)], near), \
                f"head {gi} level {lv}: saved scores of nodes outside the frontier"
            ns = rec[f"near_scores_l{lv}_g{gi}"].astype(np.float64)
            err = np.max(np.abs(ns - s_ref[pos])) if len(pos) else 0.0
            assert err <= P.SCORE_TOL, f"head {gi} level {lv}: score error {err:.3e}"
            s_gpu = s_ref.copy()
            s_gpu[pos] = ns
            kept = rec[f"kept_l{lv}_g{gi}"].astype(np.int64)
            sel = P.check_selection(fr, s_ref, s_gpu, kept, p)
            assert not sel["bad"], f"head {gi} level {lv}: {sel['bad'][:4]}"
            rep["selections"] += 1
            rep["band"] += len(sel["band"])
            rep["swap"] += len(sel["swap"])
            prev = kept
        blocks = rec[f"blocks_g{gi}"].astype(np.int64)
        assert np.array_equal(blocks, prev), f"head {gi}: gathered blocks != kept level-1 nodes"
        rep["same"] = rep["band"] == 0 and rep["swap"] == 0
        if rep["same"]:
            route = zo.route(tree, q, p)
            for lr in route["levels"]:
                assert np.array_equal(lr["kept"], rec[f"kept_l{lr['level']}_g{gi}"]), \
                    f"head {gi} level {lr['level']}: kept set differs from the oracle's route"
        tok = (blocks[:, None] * b + np.arange(b)[None, :]).ravel()
        tokens[gi] = np.union1d([0], tok[tok < n])
        reps.append(rep)
    P.assert_exemption_rates("ultra 16M KV head 0, oracle tree", reps)
    # values of the gathered tokens, chunk by chunk
    need = np.unique(np.concatenate(list(tokens.values())))
    vals = np.empty((len(need), w.head_dim), np.float64)
    for lo in range(0, n, gen.CHUNK):
        hi = min(n, lo + gen.CHUNK)
        a, z = np.searchsorted(need, [lo, hi])
        if a < z:
            vals[a:z] = gen.token_rows(w, gen.STREAM_V, 0, lo, hi)[need[a:z] - lo]
    for gi in range(w.group):
        idx = np.searchsorted(need, tokens[gi])
        o_ref = zo.attend(rows_of(kbits, tokens[gi]), vals[idx], rec["q"][gi].astype(np.float64),
                          np.arange(len(idx)))
        err = P.out_err(rec["o"][gi], o_ref)
        assert err <= P.OUT_RTOL, f"head {gi}: output error {err:.3e}"
