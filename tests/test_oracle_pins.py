"""CPU tests: the oracle against what the pages and mathematics fix (no GPU needed)."""
from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest

import pins
from oracle import zha_oracle as zo
from workloads import configs as wc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("check", pins.ALL, ids=lambda f: f.__name__)
def test_pin(check):
    ok, detail = check()
    assert ok, detail


def test_geometry_from_pages():
    """Blog post, "Building the tree": with block 4, one level summarises 4 raw keys, two
    levels 16 and six levels a 4,096-token region (fixture cites the page)."""
    with open(os.path.join(GOLDEN, "geometry.json")) as f:
        g = json.load(f)
    b = g["block"]
    n = 5000
    tree = zo.Tree(keys=np.zeros((n, 1)), refs=np.zeros((1, 1)), block=b, n_levels=6, n_tokens=n, levels=[])
    for lv, tokens in g["span_tokens"].items():
        assert b ** int(lv) == tokens
        # a node at that level covers exactly that many tokens (all full nodes)
        assert tree.nodes(int(lv)) == -(-n // tokens)


def test_workload_geometry():
    """Top-level node counts of the named workloads."""
    assert wc.DEEP.nodes(6) == 64 and wc.DEEP.block ** 6 == 4096
    assert wc.WIDE.nodes(1) == 1024
    assert wc.ULTRA.nodes(7) == 8 and wc.ULTRA.nodes(1) == 2_097_152
    assert wc.TINY.block ** 3 == 64
    assert [wc.light(n).levels for n in wc.LIGHT_SIZES] == [2, 3, 3, 4, 4]
    for n in wc.LIGHT_SIZES:
        lw = wc.light(n)
        assert lw.nodes(lw.levels) <= 512 < lw.nodes(lw.levels - 1)


def test_tiny_golden():
    """The tiny workload's routed sets and outputs, as stored by tests/golden/make_golden.py
    (a script that calls only the oracle): guards the oracle against unnoticed changes."""
    import sys
    sys.path.insert(0, GOLDEN)
    import make_golden as mg
    exp = mg.load()
    got = mg.compute()
    for e, g in zip(exp["queries"], got["queries"]):
        assert e["tokens"] == g["tokens"]
        for le, lg in zip(e["levels"], g["levels"]):
            assert le["kept"] == lg["kept"]
        np.testing.assert_allclose(g["out"], e["out"], rtol=0, atol=1e-12)


def test_top_p_edge_cases():
    # empty frontier
    assert zo.top_p(np.zeros(0, np.int64), np.zeros(0), 0.9)["k"] == 0
    # single node always kept
    assert list(zo.top_p(np.array([7]), np.array([-3.0]), 0.1)["kept"]) == [7]
    # equal scores: lowest ids first
    sel = zo.top_p(np.array([5, 2, 9, 4]), np.zeros(4), 0.5)
    assert list(sel["kept"]) == [2, 4]
    # p = 1 keeps everything even with negligible masses
    sel = zo.top_p(np.arange(3), np.array([0.0, -800.0, -900.0]), 1.0)
    assert sel["k"] == 3


def test_route_tiny_tree_edge_cases():
    rng = np.random.default_rng(11)
    d = 8
    keys = rng.standard_normal((1, d))
    refs = rng.standard_normal((2, d))
    t = zo.build_tree(keys, refs, 4, 3, 1)          # a single token: every level one node
    r = zo.route(t, rng.standard_normal(d), 0.5)
    assert list(r["tokens"]) == [0]
    assert [len(lv["frontier"]) for lv in r["levels"]] == [1, 1, 1]


# ---------------------------------------------------------------- planted mistakes
# Each mutation breaks the oracle in a plausible way; at least one pin must catch it.
def _mut_level1_offset(orig):
    def f(keys, refs, block):
        s, c = orig(keys, refs, block)
        return s, c + 0.05
    return f


def _mut_parent_unweighted(orig):
    def f(s_child, c_child, refs, block):
        s, c = orig(s_child, c_child, refs, block)
        nc = s_child.shape[0]
        npar = s.shape[0]
        mean = np.stack([s_child[i * block:min((i + 1) * block, nc)].mean(axis=0) for i in range(npar)])
        return mean, c
    return f


def _mut_parent_max_not_lse(orig):
    def f(s_child, c_child, refs, block):
        s, c = orig(s_child, c_child, refs, block)
        return s, c - 0.3
    return f


def _mut_top_p_extra(orig):
    def f(frontier, scores, p):
        sel = orig(frontier, scores, p)
        k = min(sel["k"] + 1, len(frontier))
        sel = dict(sel, k=k, kept=np.sort(np.asarray(frontier)[sel["order"][:k]]))
        return sel
    return f


def _mut_route_no_sink(orig):
    def f(tree, q, p, keep_sink=True):
        return orig(tree, q, p, False)
    return f


def _mut_attend_unscaled(orig):
    def f(keys, values, q, tokens):
        return orig(keys, values, np.asarray(q) * np.sqrt(len(q)), tokens)
    return f


def _mut_scores_mean(orig):
    def f(tree, level, nodes, q):
        s, c = tree.levels[level - 1]
        sig = 1 / np.sqrt(len(q))
        return np.mean(sig * (s[nodes] @ q) + c[nodes], axis=1)
    return f


def _mut_children_shift(orig):
    def f(tree, level, nodes):
        ch = orig(tree, level, nodes) + 1
        return ch[ch < tree.nodes(level - 1)]
    return f


def _mut_bf16_truncate(orig):
    def f(x):
        x = np.asarray(x, dtype=np.float64)
        m, e = np.frexp(x)
        return np.ldexp(np.trunc(np.ldexp(m, 8)), e - 8)
    return f


def _mut_quantise_offsets(orig):
    def f(tree, levels, fmt="bf16"):
        qt = orig(tree, levels, fmt)
        qt.levels = [(s, zo.bf16_round(c)) for s, c in qt.levels]
        return qt
    return f


def _mut_quantise_next_level(orig):
    def f(tree, levels, fmt="bf16"):
        return orig(tree, [lv + 1 for lv in levels if lv < tree.n_levels], fmt)
    return f


def _mut_mxfp4_scale_low(orig):
    # the block scale one power of two too small (amax / X in [8, 16): large values clamp)
    def f(x):
        x = np.asarray(x, dtype=np.float64)
        xb = x.reshape(-1, zo.MX_BLOCK)
        amax = np.max(np.abs(xb), axis=1)
        _, e = np.frexp(amax)
        sc = np.where(amax > 0, np.ldexp(1.0, e - 1 - 3), 1.0)[:, None]
        a = np.abs(xb) / sc
        idx = np.argmin(np.abs(a[..., None] - zo.E2M1), axis=-1)
        return (np.sign(xb) * zo.E2M1[idx] * sc).reshape(x.shape)
    return f


def _mut_mxfp4_ties_away(orig):
    # halfway cases rounded away from zero (the input nudged outward before rounding)
    def f(x):
        return orig(np.asarray(x, dtype=np.float64) * (1 + 1e-12))
    return f


def _mut_level_p_shift(orig):
    def f(p, level):
        return orig(p, min(level + 1, len(p))) if np.ndim(p) else orig(p, level)
    return f


def _mut_fit_grad_sign(orig):
    def f(keys, refs, block, levels, n_tokens, queries):
        loss, g = orig(keys, refs, block, levels, n_tokens, queries)
        return loss, -g
    return f


def _mut_fit_grad_level1_only(orig):
    def f(keys, refs, block, levels, n_tokens, queries):
        loss, _ = orig(keys, refs, block, levels, n_tokens, queries)
        _, g1 = orig(keys, refs, block, 1, n_tokens, queries)
        return loss, g1
    return f


def _mut_fit_loss_reversed(orig):
    def f(keys, refs, block, levels, n_tokens, queries):
        tree = zo.build_tree(keys, refs, block, levels, n_tokens)
        total = 0.0
        for q in np.asarray(queries, dtype=np.float64):
            for lv in range(1, levels + 1):
                logm = zo.node_log_mass(keys, q, block, lv, n_tokens)
                logpi, _ = zo.router_log_probs(tree, lv, q)
                total += float(np.sum(np.exp(logpi) * (logpi - logm)))
        return total / len(queries)
    return f


def _mut_node_mass_unnormalised(orig):
    def f(keys, q, block, level, n_tokens):
        z = np.asarray(keys, dtype=np.float64)[:n_tokens] @ np.asarray(q, dtype=np.float64) / math.sqrt(len(q))
        return orig(keys, q, block, level, n_tokens) + float(np.max(z))
    return f


def _mut_router_first_plane(orig):
    def f(tree, level, q):
        s, c = tree.levels[level - 1]
        q = np.asarray(q, dtype=np.float64)
        sc = (s[:, 0, :] @ q) / math.sqrt(q.shape[0]) + c[:, 0]
        lp = sc - np.log(np.sum(np.exp(sc - sc.max()))) - sc.max()
        return lp, np.zeros(sc.shape[0], dtype=np.int64)
    return f


def _mut_dense_gqa_modulo(orig):
    def f(keys, values, q, n_tokens):
        hq = q.shape[0]
        hkv = keys.shape[0]
        tok = np.arange(n_tokens)
        return np.stack([zo.attend(keys[h % hkv], values[h % hkv], q[h], tok) for h in range(hq)])
    return f


def _mut_dense_all_rows(orig):
    def f(keys, values, q, n_tokens):
        return orig(keys, values, q, keys.shape[1])
    return f


MUTATIONS = [
    ("level1_planes", _mut_level1_offset),
    ("parent_planes", _mut_parent_unweighted),
    ("parent_planes", _mut_parent_max_not_lse),
    ("top_p", _mut_top_p_extra),
    ("route", _mut_route_no_sink),
    ("attend", _mut_attend_unscaled),
    ("node_scores", _mut_scores_mean),
    ("children", _mut_children_shift),
    ("bf16_round", _mut_bf16_truncate),
    ("quantise_planes", _mut_quantise_offsets),
    ("quantise_planes", _mut_quantise_next_level),
    ("level_p", _mut_level_p_shift),
    ("mxfp4_round", _mut_mxfp4_scale_low),
    ("mxfp4_round", _mut_mxfp4_ties_away),
    ("fit_grad", _mut_fit_grad_sign),
    ("fit_grad", _mut_fit_grad_level1_only),
    ("fit_loss", _mut_fit_loss_reversed),
    ("node_log_mass", _mut_node_mass_unnormalised),
    ("router_log_probs", _mut_router_first_plane),
    ("dense_decode", _mut_dense_gqa_modulo),
    ("dense_decode", _mut_dense_all_rows),
]


@pytest.mark.parametrize("name,mut", MUTATIONS, ids=[f"{n}-{m.__name__}" for n, m in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, name, mut):
    monkeypatch.setattr(zo, name, mut(getattr(zo, name)))
    caught = [c.__name__ for c in pins.ALL if not c()[0]]
    assert caught, f"mutation of {name} passed every pin"


def test_chunked_generation_matches_whole():
    """The chunked K/V stream used for large caches yields the same values as the whole-
    cache generator (inputs are identical on both sides of every comparison)."""
    from workloads import gen
    w = wc.DEEP.with_(n_tokens=3000, steps=2)
    K, V = gen.kv_cache(w)
    seen = 0
    for s, h, lo, hi, rows in gen.iter_kv_chunks(w):
        assert np.array_equal((K if s == gen.STREAM_K else V)[h, lo:hi], rows)
        seen += hi - lo
    assert seen == 2 * w.num_kv_heads * w.capacity
