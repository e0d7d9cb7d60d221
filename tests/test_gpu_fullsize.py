"""GPU parity at the benchmark's full sizes, through the C ABI, in the launch configuration
bench.py times (the library picks grids from the token count alone).

* deep (256K, 6 levels, R 16) and wide (256K, 1 level, R 16): one append+decode step
  compared end to end with the oracle (full oracle trees), plus the routing chain checks.
* light sweep sizes (32K..1M, R 1): end to end for one step each.
* ultra (16M tokens): sampled checks that the oracle can compute one by one —
  planes of sampled nodes (oracle built from each node's own span), scores of sampled
  frontier nodes, the top-p decision re-derived by the oracle from the GPU's own scores at
  every level, the frontier = children-of-kept chain, and attention over the GPU's gathered
  set for every query head.
Tolerances: tests/parity.py.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import parity as P
from oracle import zha_oracle as zo
from workloads import configs as wc, gen

pytestmark = pytest.mark.gpu


def upload_chunked(w):
    dt = P.torch_dtype(w)
    Kd = torch.empty(w.num_kv_heads, w.capacity, w.head_dim, dtype=dt, device="cuda")
    Vd = torch.empty_like(Kd)
    for s, h, lo, hi, rows in gen.iter_kv_chunks(w):
        (Kd if s == gen.STREAM_K else Vd)[h, lo:hi] = torch.from_numpy(rows).to(dt).cuda()
    return Kd, Vd


def fetch_rows(Kd):
    return lambda kv, idx: Kd[kv, torch.as_tensor(np.asarray(idx), device="cuda")].float().cpu().numpy()


def check_chain(w, t, q, n):
    """Per query head, on the GPU's own scores: frontier(l-1) = existing children of
    kept(l); kept(l) = the top-p (oracle arithmetic, fp64 masses) of the GPU's scores of its
    frontier, up to the mass band; the gather list = the kept level-1 blocks.  (The scores
    themselves are checked against the oracle separately.)"""
    g, b = w.group, w.block
    traces = {lv: t.trace(lv) for lv in range(0, w.levels + 1)}
    band = sel_count = 0
    for h in range(w.num_q_heads):
        kv, gi = divmod(h, g)
        prev_kept = None
        for lv in range(w.levels, 0, -1):
            tr = traces[lv][kv]
            fr = P.gpu_frontier(tr, gi)
            if prev_kept is not None:
                ch = (prev_kept[:, None] * b + np.arange(b)[None, :]).ravel()
                ch = ch[ch < w.nodes(lv, n)]
                assert np.array_equal(np.sort(ch), fr), f"head {h} level {lv}: frontier != children of kept"
            else:
                assert np.array_equal(fr, np.arange(w.nodes(lv, n))), f"head {h}: top frontier"
            s_fr = P.gpu_scores_on(tr, gi, fr)
            kept = P.gpu_kept(tr, gi)
            sel = P.check_selection(fr, s_fr, s_fr, kept, zo.level_p(w.top_p, lv))
            assert not sel["bad"], f"head {h} level {lv}: kept set is not the top-p of the GPU scores: {sel['bad'][:4]}"
            band += len(sel["band"])
            sel_count += 1
            prev_kept = kept
        blocks = P.gpu_frontier(traces[0][kv], gi)
        assert np.array_equal(blocks, prev_kept), f"head {h}: gather list != kept level-1 blocks"
    P.assert_exemption_rates(f"{w.name} chain on the GPU scores", dict(bad=[], band=band, swap=0, selections=sel_count))
    return traces


def attention_given_set(w, traces, o, q, n, Kd, Vd, heads):
    for h in heads:
        kv, gi = divmod(h, w.group)
        toks = P.gpu_tokens(traces[0][kv], gi, w.block, n, w.keep_sink)
        tk = torch.as_tensor(toks, device="cuda")
        k = Kd[kv, tk].double().cpu().numpy()
        v = Vd[kv, tk].double().cpu().numpy()
        ref = zo.attend(k, v, q[h], np.arange(len(toks)))
        err = P.out_err(o[h], ref)
        assert err <= P.OUT_RTOL, f"head {h}: attention over the routed set err {err:.3e}"


@pytest.mark.parametrize("name,planes", [("deep", "f32"), ("wide", "f32"), ("deep", "bf16"), ("deep", "fp4")])
def test_256k_end_to_end(name, planes):
    w = wc.NAMED[name].with_(steps=1, planes=planes)
    K, V = gen.kv_cache(w)
    refs = gen.ref_queries(w)
    Kd, Vd = P.upload(K, w), P.upload(V, w)
    t = P.make_tree(w)
    if planes != "f32":
        t.set_route_mode(1)    # the union frontiers, which read the quantised plane copies
    t.build(Kd, Vd, w.n_tokens, P.upload(refs, w))
    t.append(Kd[:, w.n_tokens].contiguous(), Vd[:, w.n_tokens].contiguous())
    n = w.n_tokens + 1
    q = gen.step_queries(w, 0, n, gen.host_fetch(K))
    o = t.decode(P.upload(q, w)).cpu().numpy()
    traces = check_chain(w, t, q, n)
    attention_given_set(w, traces, o, q, n, Kd, Vd, range(w.num_q_heads))
    # full oracle, end to end (quantised router planes: the oracle's quantisation, with the
    # rounding-flip allowance in the score tolerance)
    trees = P.oracle_trees(w, K, refs, n)
    tol_fn = lambda kv, qh: (lambda lv, fr: P.SCORE_TOL + P.flip_allowance(w, trees[kv], lv, fr, qh))
    reps = P.check_decode(P.router_trees(w, trees), K, V, q, o, traces, w.top_p, w.keep_sink, n, tol_fn=tol_fn)
    P.assert_exemption_rates(f"{name} {planes} 256K end to end", reps)
    if planes != "f32":
        t.close()
        return
    # dense decode at full size
    od = t.decode_dense(P.upload(q, w)).cpu().numpy()
    ref_d = zo.dense_decode(K, V, q, n)
    assert P.out_err(od, ref_d) <= P.OUT_RTOL


@pytest.mark.parametrize("n_tokens", wc.LIGHT_SIZES)
def test_light_sweep_end_to_end(n_tokens):
    w = wc.light(n_tokens, steps=1)
    K, V = gen.kv_cache(w)
    refs = gen.ref_queries(w)
    Kd, Vd = P.upload(K, w), P.upload(V, w)
    t = P.make_tree(w)
    t.build(Kd, Vd, w.n_tokens, P.upload(refs, w))
    t.append(Kd[:, w.n_tokens].contiguous(), Vd[:, w.n_tokens].contiguous())
    n = w.n_tokens + 1
    q = gen.step_queries(w, 0, n, gen.host_fetch(K))
    o = t.decode(P.upload(q, w)).cpu().numpy()
    traces = check_chain(w, t, q, n)
    trees = P.oracle_trees(w, K, refs, n)
    reps = P.check_decode(trees, K, V, q, o, traces, w.top_p, w.keep_sink, n)
    P.assert_exemption_rates(f"light {n_tokens} end to end", reps)


@pytest.mark.parametrize("planes", ["f32", "fp4"])
def test_ultra_16m_sampled(planes):
    w = wc.ULTRA.with_(steps=1, planes=planes)
    Kd, Vd = upload_chunked(w)
    refs = gen.ref_queries(w)
    t = P.make_tree(w)
    t.build(Kd, Vd, w.n_tokens, P.upload(refs, w))
    t.append(Kd[:, w.n_tokens].contiguous(), Vd[:, w.n_tokens].contiguous())
    n = w.n_tokens + 1
    q = gen.step_queries(w, 0, n, fetch_rows(Kd))
    o = t.decode(P.upload(q, w)).cpu().numpy()
    traces = check_chain(w, t, q, n)
    attention_given_set(w, traces, o, q, n, Kd, Vd, range(w.num_q_heads))
    # sampled planes and scores against the oracle, per level, computed from node spans
    rng = np.random.default_rng(0)
    sig = 1.0 / math.sqrt(w.head_dim)
    for lv in range(1, w.levels + 1):
        s_gpu, c_gpu = t.level(lv)
        nl = w.nodes(lv, n)
        span = w.block ** lv
        picks = sorted(set(rng.integers(0, nl, 3).tolist()) | {nl - 1})
        if span > 300_000:
            picks = [nl - 1]
        for kv in range(w.num_kv_heads):
            tr = traces[lv][kv]
            tnodes = tr["nodes"].numpy().astype(np.int64)
            for node in picks:
                lo, hi = node * span, min((node + 1) * span, n)
                keys = Kd[kv, lo:hi].double().cpu().numpy()
                ot = zo.build_tree(keys, refs[kv], w.block, lv, hi - lo)
                so, co = ot.levels[lv - 1][0][0], ot.levels[lv - 1][1][0]
                sg, cg = s_gpu[kv, node].cpu().numpy(), c_gpu[kv, node].cpu().numpy()
                assert np.max(np.abs(sg - so)) <= 1e-4 * max(1.0, np.max(np.abs(so))), f"s level {lv} node {node}"
                assert np.max(np.abs(cg - co)) <= 1e-3, f"c level {lv} node {node}"
                pos = int(np.searchsorted(tnodes, node))
                if pos < len(tnodes) and tnodes[pos] == node:
                    routed = planes != "f32" and lv in P.router_levels(w)
                    sr = zo.QUANTISERS[planes](so) if routed else so
                    mk = int(tr["masks"][pos]) & 0xFFFFFFFF
                    for g_ in range(w.group):
                        if not (mk >> g_) & 1:
                            continue        # scores exist for the heads whose frontier holds it
                        qh = q[kv * w.group + g_]
                        ref = float(np.max(sig * (sr @ qh) + co))
                        tol = P.SCORE_TOL
                        if routed:
                            lo_, hi_ = P.quant_bounds(planes, so)
                            tol += float(np.max((hi_ - lo_) @ np.abs(qh))) * sig
                        got = float(tr["scores"][g_][pos])
                        assert abs(got - ref) <= tol, f"score level {lv} node {node}: {got} vs {ref}"
