"""Property checks that pin the CPU oracle to facts outside itself.

Each check returns (ok, detail).  They are used by test_oracle_pins.py on the oracle as
written, and by the mutation tests on deliberately broken copies of it, which must fail
at least one check.  None of them re-types the oracle's own formulas: they compare with
closed forms (logsumexp / softmax over a node's whole span via SciPy), textbook routines
(torch scaled_dot_product_attention), brute force, and the geometry the pages state.
"""
from __future__ import annotations

import itertools
import math

import numpy as np
import scipy.special as sp
import torch

from oracle import zha_oracle as zo


def rand_tree(rng, n=203, d=8, r=3, b=4, levels=3, scale=1.0):
    keys = rng.standard_normal((n, d)) * scale
    refs = rng.standard_normal((r, d))
    return zo.build_tree(keys, refs, b, levels, n), keys, refs


def span(tree, level, node):
    b = tree.block ** level
    return np.arange(node * b, min((node + 1) * b, tree.n_tokens))


def true_lse(keys, q, toks):
    return sp.logsumexp(keys[toks] @ q / math.sqrt(q.shape[0]))


# P2: every plane (hence the max over planes) lower-bounds the node's true log mass.
def check_convexity(seed=0, n_q=20):
    rng = np.random.default_rng(seed)
    tree, keys, _ = rand_tree(rng)
    worst = -np.inf
    for lv in range(1, tree.n_levels + 1):
        nodes = np.arange(tree.nodes(lv))
        for _ in range(n_q):
            q = rng.standard_normal(keys.shape[1]) * 3
            sc = zo.node_scores(tree, lv, nodes, q)
            tl = np.array([true_lse(keys, q, span(tree, lv, n)) for n in nodes])
            worst = max(worst, np.max(sc - tl - 1e-12 * np.maximum(1, np.abs(tl))))
    return worst <= 0, f"max(score - true LSE) = {worst:.3e}"


# P3: plane j is exact at q = r_j (level 1 required; every level by the recursion).
def check_exact_at_refs(seed=1):
    rng = np.random.default_rng(seed)
    tree, keys, refs = rand_tree(rng)
    d = keys.shape[1]
    worst = 0.0
    for lv in range(1, tree.n_levels + 1):
        s, c = tree.levels[lv - 1]
        for n in range(tree.nodes(lv)):
            for j in range(refs.shape[0]):
                plane = refs[j] @ s[n, j] / math.sqrt(d) + c[n, j]
                score = zo.node_scores(tree, lv, np.array([n]), refs[j])[0]
                tl = true_lse(keys, refs[j], span(tree, lv, n))
                worst = max(worst, abs(plane - tl), abs(score - tl))
    return worst < 1e-10, f"max |plane_j(r_j) - LSE_j| = {worst:.3e}"


# P4: recursion equals the direct per-span definition (softmax-weighted mean key, LSE).
def check_recursion_direct(seed=2):
    rng = np.random.default_rng(seed)
    tree, keys, refs = rand_tree(rng, n=300, b=3, levels=4)
    d = keys.shape[1]
    worst = 0.0
    for lv in range(1, tree.n_levels + 1):
        s, c = tree.levels[lv - 1]
        for n in range(tree.nodes(lv)):
            toks = span(tree, lv, n)
            for j in range(refs.shape[0]):
                z = keys[toks] @ refs[j] / math.sqrt(d)
                w = sp.softmax(z)
                s_dir = w @ keys[toks]
                lse_dir = sp.logsumexp(z)
                lse = c[n, j] + refs[j] @ s[n, j] / math.sqrt(d)
                worst = max(worst, np.max(np.abs(s[n, j] - s_dir)), abs(lse - lse_dir))
    return worst < 1e-10, f"max |recursive - direct| = {worst:.3e}"


# R20: every node's router score follows from the keys upwards.  With D_j = sigma q.s_j, a
# level-1 node's D_j is its keys' sigma q.k_t weighted by exp(sigma r_j.k_t - LSE_j), and a
# parent's is its children's D_j weighted by exp(LSE_cj - LSE_j); max_j (D_j + c_j) is then
# the plane score at every level.  (LSE_j is recovered from the planes as c_j + sigma r_j.s_j.)
def check_scores_from_keys(seed=21):
    rng = np.random.default_rng(seed)
    tree, keys, refs = rand_tree(rng, n=1001, d=8, r=4, b=4, levels=4)
    sig = 1.0 / math.sqrt(keys.shape[1])
    q = rng.standard_normal(keys.shape[1]) * 2.0
    worst = 0.0
    d_below = lse_below = None
    for lv in range(1, tree.n_levels + 1):
        s, c = tree.levels[lv - 1]
        lse = c + sig * np.einsum("njd,jd->nj", s, refs)
        nn = tree.nodes(lv)
        dots = np.zeros((nn, refs.shape[0]))
        for n in range(nn):
            if lv == 1:
                toks = span(tree, 1, n)
                w = np.exp(sig * keys[toks] @ refs.T - lse[n])            # [tokens, R]
                dots[n] = w.T @ (sig * keys[toks] @ q)
            else:
                ch = np.arange(n * tree.block, min((n + 1) * tree.block, tree.nodes(lv - 1)))
                dots[n] = np.sum(np.exp(lse_below[ch] - lse[n]) * d_below[ch], axis=0)
        score = np.max(dots + c, axis=1)
        worst = max(worst, np.max(np.abs(score - zo.node_scores(tree, lv, np.arange(nn), q))))
        d_below, lse_below = dots, lse
    return worst < 1e-9, f"max |score from the keys - plane score| = {worst:.3e}"


# P5: single-key nodes are exact: s_j = k, c_j = 0, score = sigma q.k.
def check_single_key(seed=3):
    rng = np.random.default_rng(seed)
    d = 8
    keys = rng.standard_normal((37, d))
    refs = rng.standard_normal((3, d))
    t1 = zo.build_tree(keys, refs, 1, 1, 37)           # b = 1: every block one key
    t4 = zo.build_tree(keys, refs, 4, 1, 37)           # last block of b = 4 holds one key
    q = rng.standard_normal(d)
    s1, c1 = t1.levels[0]
    worst = max(np.max(np.abs(s1 - keys[:, None, :])), np.max(np.abs(c1)))
    sc = zo.node_scores(t1, 1, np.arange(37), q)
    worst = max(worst, np.max(np.abs(sc - keys @ q / math.sqrt(d))))
    s4, c4 = t4.levels[0]
    worst = max(worst, np.max(np.abs(s4[-1] - keys[36])), np.max(np.abs(c4[-1])))
    return worst < 1e-12, f"max single-key error = {worst:.3e}"


# P6: b = 1, L = 1 is textbook nucleus selection over the true attention distribution.
def check_nucleus(seed=4, p=0.8):
    rng = np.random.default_rng(seed)
    d, n = 16, 200
    keys = rng.standard_normal((n, d))
    refs = rng.standard_normal((2, d))
    tree = zo.build_tree(keys, refs, 1, 1, n)
    bad = 0
    for _ in range(10):
        q = rng.standard_normal(d) * 4
        probs = sp.softmax(keys @ q / math.sqrt(d))
        idx = np.argsort(-probs, kind="stable")
        k = int(np.searchsorted(np.cumsum(probs[idx]), p)) + 1
        expect = np.union1d([0], idx[:k])
        got = zo.route(tree, q, p)["tokens"]
        bad += not np.array_equal(np.sort(expect), got)
    return bad == 0, f"{bad} of 10 queries differ from nucleus selection"


# P7: the kept set is minimal (brute force over all subsets) and heaviest among minimal sets.
def check_minimal(seed=5, trials=40):
    rng = np.random.default_rng(seed)
    fails = 0
    for t in range(trials):
        f = int(rng.integers(1, 13))
        scores = rng.standard_normal(f) * rng.uniform(0.1, 4)
        if t % 5 == 0:
            scores = np.round(scores)                     # force ties
        frontier = np.sort(rng.choice(1000, size=f, replace=False))
        p = float(rng.choice([0.3, 0.75, 0.95, 0.999, 1.0]))
        probs = sp.softmax(scores)
        best_k, best_mass = None, -1.0
        for k in range(1, f + 1):
            masses = [probs[list(c)].sum() for c in itertools.combinations(range(f), k)]
            mx = max(masses)
            if p >= 1.0:
                if k == f:
                    best_k, best_mass = k, mx
            elif mx >= p - 1e-12:
                best_k, best_mass = k, mx
                break
        sel = zo.top_p(frontier, scores, p)
        kept_mass = probs[np.isin(frontier, sel["kept"])].sum()
        if sel["k"] != best_k or abs(kept_mass - best_mass) > 1e-12:
            fails += 1
    return fails == 0, f"{fails} of {trials} frontiers not minimal/heaviest"


# P8: mass conservation at every level.
def check_mass_conservation(seed=6):
    rng = np.random.default_rng(seed)
    tree, keys, refs = rand_tree(rng, n=259, b=4, levels=4)
    d = keys.shape[1]
    worst = 0.0
    for lv in range(1, tree.n_levels + 1):
        s, c = tree.levels[lv - 1]
        lse = c + np.einsum("nrd,rd->nr", s, refs) / math.sqrt(d)
        for j in range(refs.shape[0]):
            z = keys @ refs[j] / math.sqrt(d)
            a = sp.logsumexp(lse[:, j])
            b = sp.logsumexp(z)
            m1 = np.exp(lse[:, j] - b) @ s[:, j]
            m2 = np.exp(z - b) @ keys
            worst = max(worst, abs(a - b), np.max(np.abs(m1 - m2)))
    return worst < 1e-10, f"max conservation error = {worst:.3e}"


# P9: build(N) + m appends equals build(N + m).
def check_append(seed=7, n0=61, m=70, b=4, levels=4):
    rng = np.random.default_rng(seed)
    d = 8
    keys = rng.standard_normal((n0 + m, d))
    refs = rng.standard_normal((3, d))
    t = zo.build_tree(keys.copy(), refs, b, levels, n0)
    for i in range(m):
        zo.append_token(t, keys[n0 + i])
    full = zo.build_tree(keys, refs, b, levels, n0 + m)
    worst = 0.0
    for (sa, ca), (sb, cb) in zip(t.levels, full.levels):
        if sa.shape != sb.shape:
            return False, f"level shapes {sa.shape} vs {sb.shape}"
        worst = max(worst, np.max(np.abs(sa - sb)), np.max(np.abs(ca - cb)))
    return worst < 1e-12, f"max |append - rebuild| = {worst:.3e}"


def _sdpa(keys, values, q, mask=None):
    qt = torch.from_numpy(np.asarray(q, np.float64))[None, None, None, :]
    kt = torch.from_numpy(np.asarray(keys, np.float64))[None, None]
    vt = torch.from_numpy(np.asarray(values, np.float64))[None, None]
    m = None if mask is None else torch.from_numpy(mask)[None, None, None, :]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m)[0, 0, 0].numpy()


# P1: p = 1 reproduces dense attention (torch SDPA, float64 on the CPU).
def check_dense_limit(seed=8):
    rng = np.random.default_rng(seed)
    hkv, hq, d, n = 2, 6, 16, 301
    keys = rng.standard_normal((hkv, n, d))
    vals = rng.standard_normal((hkv, n, d))
    refs = rng.standard_normal((hkv, 3, d))
    trees = [zo.build_tree(keys[h], refs[h], 4, 3, n) for h in range(hkv)]
    q = rng.standard_normal((hq, d)) * 3
    o = zo.decode(trees, vals, q, 1.0)
    g = hq // hkv
    ref = np.stack([_sdpa(keys[h // g], vals[h // g], q[h]) for h in range(hq)])
    err = np.max(np.abs(o - ref))
    return err < 1e-12, f"max |ZHA(p=1) - SDPA| = {err:.3e}"


# Dense decode (the crossover baseline): every query head against torch SDPA over all n
# tokens of its KV head, under the contiguous GQA mapping (query head h reads KV head
# h // (Hq / Hkv)).  The caches hold rows past n that must not be attended.
def check_dense_decode(seed=20):
    rng = np.random.default_rng(seed)
    hkv, hq, d, n, cap = 2, 6, 16, 131, 140
    keys = rng.standard_normal((hkv, cap, d))
    vals = rng.standard_normal((hkv, cap, d))
    q = rng.standard_normal((hq, d)) * 3
    o = zo.dense_decode(keys, vals, q, n)
    g = hq // hkv
    ref = np.stack([_sdpa(keys[h // g][:n], vals[h // g][:n], q[h]) for h in range(hq)])
    err = np.max(np.abs(o - ref))
    return err < 1e-12, f"max |dense_decode - SDPA per head| = {err:.3e}"


# P11: attention over a given set equals masked dense attention.
def check_masked_attention(seed=9):
    rng = np.random.default_rng(seed)
    d, n = 16, 97
    keys = rng.standard_normal((n, d))
    vals = rng.standard_normal((n, d))
    q = rng.standard_normal(d) * 2
    toks = np.union1d([0], rng.choice(n, 30, replace=False))
    mask = np.zeros(n, bool)
    mask[toks] = True
    err = np.max(np.abs(zo.attend(keys, vals, q, toks) - _sdpa(keys, vals, q, mask)))
    return err < 1e-12, f"max |attend(S) - masked SDPA| = {err:.3e}"


# Sink: token 0 is always attended, and only once.
def check_sink(seed=10):
    rng = np.random.default_rng(seed)
    tree, keys, _ = rand_tree(rng, n=400)
    ok = True
    for _ in range(10):
        q = rng.standard_normal(keys.shape[1]) * 4
        toks = zo.route(tree, q, 0.5)["tokens"]
        ok &= toks[0] == 0 and np.unique(toks).size == toks.size
    return bool(ok), "sink present and unique"


# bf16 router planes.  Rounding of float32 inputs = torch's float32 -> bfloat16 cast
# (round to nearest, ties to even), including values exactly halfway between two
# bfloat16 neighbours with either parity of the kept last bit.
def check_bf16_round_library(seed=11):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    hi = rng.integers(0x3000, 0x4f00, 4000, dtype=np.uint32)
    half = ((hi << 16) | 0x8000).astype(np.uint32)
    half = np.concatenate([half, half | np.uint32(0x80000000)]).view(np.float32)
    x = np.concatenate([x, half, np.array([0.0, 1.0, -2.5, 3.0e-30], np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = zo.bf16_round(x.astype(np.float64))
    bad = int(np.count_nonzero(got != want))
    return bad == 0, f"{bad} of {x.size} roundings differ from torch's cast"


# Rounding of float64 inputs = the nearest of all finite bfloat16 values, by brute force
# over every bit pattern; exact midpoints of neighbours go to the even pattern.
def check_bf16_round_nearest(seed=12):
    rng = np.random.default_rng(seed)
    pats = np.arange(1 << 16, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        vals = (pats << 16).view(np.float32).astype(np.float64)
    fin = np.isfinite(vals) & ~((vals == 0) & (pats != 0))     # one zero
    vals, pats = vals[fin], pats[fin]
    order = np.argsort(vals, kind="stable")
    vals, pats = vals[order], pats[order]
    x = rng.standard_normal(5000) * np.exp(rng.uniform(-30, 30, 5000))
    i = np.clip(np.searchsorted(vals, x), 1, len(vals) - 1)
    lo, hi = vals[i - 1], vals[i]
    want = np.where(x - lo < hi - x, lo, hi)
    # constructed midpoints of neighbouring positive normal values
    first = int(np.searchsorted(vals, 2.0 ** -126))
    k = rng.integers(first, len(vals) - 2, 2000)
    mid = (vals[k] + vals[k + 1]) / 2
    want_mid = np.where(pats[k] % 2 == 0, vals[k], vals[k + 1])
    got, got_mid = zo.bf16_round(x), zo.bf16_round(mid)
    bad = int(np.count_nonzero(got != want)) + int(np.count_nonzero(got_mid != want_mid))
    return bad == 0, f"{bad} roundings differ from the brute-force nearest value"


# Quantised planes: the listed levels' s become bfloat16 values within half a unit
# (2^-8 |s|), the offsets and the other levels are untouched, and each node's score moves
# by at most max_j sigma * sum_i |q_i| |s~_ji - s_ji| (a max of planes moves by at most
# the largest plane move).
def check_quantised_planes(seed=13):
    rng = np.random.default_rng(seed)
    tree, keys, _ = rand_tree(rng, n=300, d=16, r=3, b=4, levels=3)
    qt = zo.quantise_planes(tree, [1, 3])
    d = keys.shape[1]
    sig = 1.0 / math.sqrt(d)
    moved = 0
    for lv in range(1, 4):
        s, c = tree.levels[lv - 1]
        sq, cq = qt.levels[lv - 1]
        if not np.array_equal(cq, c):
            return False, f"level {lv}: offsets changed"
        if lv == 2:
            if not np.array_equal(sq, s):
                return False, "level 2 (not listed) changed"
            continue
        f = torch.from_numpy(sq.astype(np.float32))
        if not (np.array_equal(f.numpy().astype(np.float64), sq) and
                torch.equal(f.to(torch.bfloat16).to(torch.float32), f)):
            return False, f"level {lv}: s is not made of bfloat16 values"
        if np.any(np.abs(sq - s) > 2.0 ** -8 * np.abs(s)):
            return False, f"level {lv}: rounding error above half a unit"
        nodes = np.arange(tree.nodes(lv))
        for _ in range(10):
            q = rng.standard_normal(d) * 3
            a = zo.node_scores(tree, lv, nodes, q)
            b = zo.node_scores(qt, lv, nodes, q)
            bound = sig * np.max(np.abs(sq - s) @ np.abs(q), axis=1)
            if np.any(np.abs(b - a) > bound * (1 + 1e-9) + 1e-15):
                return False, f"level {lv}: score moved beyond the plane bound"
            moved += int(np.count_nonzero(a != b))
    return moved > 0, f"{moved} quantised scores moved"


# Per-level p: with p = 1 at every level but one, routing reduces to a textbook nucleus
# selection at that level (over all its nodes, by softmax of their scores), and every
# level below keeps all children of the selected nodes.  Checked for the top level and
# for level 1 of a 3-level tree.
def check_p_schedule(seed=14):
    rng = np.random.default_rng(seed)
    tree, keys, _ = rand_tree(rng, n=203, d=8, r=3, b=4, levels=3)
    bad = 0
    for _ in range(10):
        q = rng.standard_normal(keys.shape[1]) * 3
        for lv, p in ((1, 0.6), (3, 0.5)):
            sched = [1.0, 1.0, 1.0]
            sched[lv - 1] = p
            nodes = np.arange(tree.nodes(lv))
            pi = sp.softmax(zo.node_scores(tree, lv, nodes, q))
            order = sorted(nodes.tolist(), key=lambda n: (-pi[n], n))
            keep, mass = [], 0.0
            for n in order:
                keep.append(n)
                mass += pi[n]
                if mass >= p:
                    break
            span_l = tree.block ** lv
            toks = {t for n in keep for t in range(n * span_l, min((n + 1) * span_l, tree.n_tokens))} | {0}
            got = zo.route(tree, q, sched)
            bad += set(got["tokens"].tolist()) != toks
    return bad == 0, f"{bad} schedules routed differently from the nucleus selection"


# FP4 router planes.  mxfp4_round against a brute-force search: per block of 32, the scale
# is the power of two X with amax / X in [4, 8) (found by doubling from 2^-40), and each
# element the nearest of the 16 codes times X (clamped at 6X), halfway cases to the even
# code; plus constructed halfway cases of every pair of neighbouring magnitudes.
def check_mxfp4_round(seed=15):
    rng = np.random.default_rng(seed)
    codes = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    bad = 0
    for _ in range(300):
        x = rng.standard_normal(32) * np.exp(rng.uniform(-8, 8))
        if rng.random() < 0.2:
            x[rng.integers(0, 32, 5)] = 0.0
        amax = np.max(np.abs(x))
        X = 2.0 ** -40
        while amax / X >= 8:
            X *= 2
        want = np.empty(32)
        for i, v in enumerate(x):
            a = min(abs(v) / X, 6.0)
            d = np.abs(codes - a)
            best = np.nonzero(d == d.min())[0]
            k = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
            want[i] = math.copysign(codes[k] * X, v)
        bad += int(np.count_nonzero(zo.mxfp4_round(x) != want))
    # halfway cases: a block with amax = 4X (X = 1/8) holding every midpoint of neighbours
    X = 0.125
    mids = (codes[:-1] + codes[1:]) / 2
    block = np.zeros(32)
    block[0] = 4 * X
    block[1:1 + len(mids)] = mids * X
    block[8:8 + len(mids)] = -mids * X
    even = np.array([codes[i] if i % 2 == 0 else codes[i + 1] for i in range(len(mids))])
    got = zo.mxfp4_round(block)
    bad += int(np.count_nonzero(got[1:1 + len(mids)] != even * X))
    bad += int(np.count_nonzero(got[8:8 + len(mids)] != -even * X))
    return bad == 0, f"{bad} elements differ from the brute-force rounding"


# FP4 planes: each block's largest quantised magnitude is 4X or 6X (amax / X in [4, 8)),
# every element moves by at most 2X, the offsets stay, and each score moves by at most the
# largest plane move, max_j sigma * sum_i |q_i| |s~_ji - s_ji|.
def check_fp4_planes(seed=16):
    rng = np.random.default_rng(seed)
    tree, keys, _ = rand_tree(rng, n=300, d=64, r=2, b=4, levels=2)
    qt = zo.quantise_planes(tree, [1, 2], "fp4")
    sig = 1.0 / math.sqrt(keys.shape[1])
    moved = 0
    for lv in (1, 2):
        s, c = tree.levels[lv - 1]
        sq, cq = qt.levels[lv - 1]
        if not np.array_equal(cq, c):
            return False, f"level {lv}: offsets changed"
        sb, qb = s.reshape(-1, 32), sq.reshape(-1, 32)
        _, e = np.frexp(np.max(np.abs(sb), axis=1))
        X = np.ldexp(1.0, e - 3)[:, None]
        top = np.max(np.abs(qb), axis=1, keepdims=True) / X
        if not np.all((top == 4) | (top == 6)):
            return False, f"level {lv}: a block's largest code is not 4 or 6"
        if np.any(np.abs(qb - sb) > 2 * X):
            return False, f"level {lv}: an element moved by more than 2X"
        nodes = np.arange(tree.nodes(lv))
        for _ in range(10):
            q = rng.standard_normal(keys.shape[1]) * 3
            a = zo.node_scores(tree, lv, nodes, q)
            b = zo.node_scores(qt, lv, nodes, q)
            bound = sig * np.max(np.abs(sq - s) @ np.abs(q), axis=1)
            if np.any(np.abs(b - a) > bound * (1 + 1e-9) + 1e-15):
                return False, f"level {lv}: score moved beyond the plane bound"
            moved += int(np.count_nonzero(a != b))
    return moved > 0, f"{moved} quantised scores moved"


# K3: the fitting gradient is the derivative of the fitting loss (central differences of
# the loss, which rebuilds the tree at every perturbed point).
def check_fit_grad_fd(seed=17):
    rng = np.random.default_rng(seed)
    worst = 0.0
    for (n, d, r, b, levels) in [(13, 8, 3, 2, 3), (37, 8, 1, 4, 2), (29, 6, 2, 3, 3)]:
        keys = rng.standard_normal((n, d))
        refs = rng.standard_normal((r, d))
        qs = rng.standard_normal((3, d)) * 2
        loss, g = zo.fit_grad(keys, refs, b, levels, n, qs)
        if abs(loss - zo.fit_loss(keys, refs, b, levels, n, qs)) > 1e-12 * max(1.0, abs(loss)):
            return False, "fit_grad's loss differs from fit_loss"
        h = 1e-6
        for i in range(r):
            for k in range(d):
                rp, rm = refs.copy(), refs.copy()
                rp[i, k] += h
                rm[i, k] -= h
                num = (zo.fit_loss(keys, rp, b, levels, n, qs) - zo.fit_loss(keys, rm, b, levels, n, qs)) / (2 * h)
                err = abs(num - g[i, k])
                worst = max(worst, err)
                if err > 1e-6 * max(1.0, abs(num)):
                    return False, f"n={n} b={b}: d loss / d r[{i},{k}] {g[i, k]:.8f} vs difference {num:.8f}"
    return True, f"worst gradient error {worst:.1e}"


# K1: the fitting loss against a brute-force KL built from closed forms: each node's score
# is the max over the reference queries of the tangent of the node's true log mass (SciPy
# logsumexp / softmax over the node's span), the router distribution is the softmax of
# those scores over the level, the target is the dense softmax summed over each span, and
# the divergence is SciPy's relative entropy of the target to the router.
def check_fit_loss_bruteforce(seed=18):
    rng = np.random.default_rng(seed)
    n, d, r, b, levels = 45, 8, 3, 3, 3
    keys = rng.standard_normal((n, d))
    refs = rng.standard_normal((r, d))
    qs = rng.standard_normal((4, d)) * 2
    sig = 1.0 / math.sqrt(d)
    total = 0.0
    for q in qs:
        dense = sp.softmax(keys @ q * sig)
        for lv in range(1, levels + 1):
            nn = -(-n // b ** lv)
            toks = [np.arange(j * b ** lv, min((j + 1) * b ** lv, n)) for j in range(nn)]
            mass = np.array([dense[t].sum() for t in toks])
            scores = []
            for t in toks:
                best = -np.inf
                for rj in refs:
                    w = sp.softmax(keys[t] @ rj * sig)
                    tangent = true_lse(keys, rj, t) + sig * (q - rj) @ (w @ keys[t])
                    best = max(best, tangent)
                scores.append(best)
            total += float(np.sum(sp.rel_entr(mass, sp.softmax(np.array(scores)))))
    want = total / len(qs)
    got = zo.fit_loss(keys, refs, b, levels, n, qs)
    if not (got >= 0.0 and abs(got - want) <= 1e-10 * max(1.0, want)):
        return False, f"loss {got:.12f} vs brute force {want:.12f}"
    return True, f"loss {got:.6f}"


# K2: single-key blocks make every tangent plane exact (the plane of one key is sigma q.k),
# so the router reproduces dense attention at every level: zero loss and zero gradient.
def check_fit_single_key(seed=19):
    rng = np.random.default_rng(seed)
    n, d = 17, 8
    keys = rng.standard_normal((n, d))
    refs = rng.standard_normal((2, d))
    qs = rng.standard_normal((3, d)) * 3
    loss, g = zo.fit_grad(keys, refs, 1, 2, n, qs)
    if abs(loss) > 1e-12 or np.max(np.abs(g)) > 1e-12:
        return False, f"b=1: loss {loss:.2e}, largest gradient {np.max(np.abs(g)):.2e}"
    loss4 = zo.fit_loss(keys, refs, 4, 2, n, qs)
    return loss4 > 1e-6, f"b=4 loss {loss4:.4f} (> 0)"


ALL = [check_dense_limit, check_dense_decode, check_convexity, check_exact_at_refs, check_recursion_direct,
       check_scores_from_keys,
       check_single_key, check_nucleus, check_minimal, check_mass_conservation, check_append,
       check_masked_attention, check_sink, check_bf16_round_library, check_bf16_round_nearest,
       check_quantised_planes, check_p_schedule, check_mxfp4_round, check_fp4_planes,
       check_fit_grad_fd, check_fit_loss_bruteforce, check_fit_single_key]
