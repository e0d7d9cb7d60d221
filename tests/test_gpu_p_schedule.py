"""GPU parity of per-level top-p schedules (zha_set_top_p_levels) against the oracle.

A schedule gives each level its own p (oracle ``level_p``).  Checked on the deep tree
(key-form level 1, top-down upper levels), the light router through the large-level path,
and the tiny fp32 tree: teacher-forced scores and sets per level, and decode end to end
after appends, with a fixed schedule and with one that changes between decodes (a
context-dependent p_l(N) set before each decode).  Tolerances: tests/parity.py.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import parity as P
from oracle import zha_oracle as zo
from workloads import configs as wc, gen

pytestmark = pytest.mark.gpu

CASES = {
    # levels 1..6
    "deep_small": (wc.DEEP.with_(n_tokens=16_384 + 37, steps=2), [0.5, 0.9, 0.97, 0.99, 1.0, 0.8]),
    # levels 1..4; level 1 (36,001 nodes) through the large-level path
    "light_general": (wc.light(288_003, steps=2).with_(num_kv_heads=1, num_q_heads=8), [0.6, 0.9, 1.0, 0.85]),
    "tiny": (wc.TINY.with_(steps=3), [0.3, 0.99, 0.9]),
}


def setup(name):
    w, sched = CASES[name]
    K, V, refs = P.host_inputs(w)
    trees = P.oracle_trees(w, K, refs, w.n_tokens)
    t = P.make_tree(w)
    Kd, Vd = P.upload(K, w), P.upload(V, w)
    t.build(Kd, Vd, w.n_tokens, P.upload(refs, w))
    t.set_top_p_levels(sched)
    return w, sched, K, V, trees, t, Kd, Vd


@pytest.mark.parametrize("name", list(CASES))
def test_teacher_forced_sets(name):
    w, sched, K, V, trees, t, _, _ = setup(name)
    g = w.group
    q = gen.step_queries(w, 100, w.n_tokens, gen.host_fetch(K))
    routes = [zo.route(trees[h // g], q[h], sched, w.keep_sink) for h in range(w.num_q_heads)]
    qd = P.upload(q, w)
    for li in range(w.levels):
        lv = w.levels - li
        fronts = []
        for kv in range(w.num_kv_heads):
            fr = {}
            for gi in range(g):
                for n in routes[kv * g + gi]["levels"][li]["frontier"].tolist():
                    fr[n] = fr.get(n, 0) | (1 << gi)
            nodes = np.array(sorted(fr), dtype=np.int64)
            fronts.append((nodes, np.array([fr[n] for n in nodes.tolist()], dtype=np.int64)))
        tr = t.route_level(lv, qd, fronts)
        for h in range(w.num_q_heads):
            kv, gi = divmod(h, g)
            rec = routes[h]["levels"][li]
            gs = P.gpu_scores(tr[kv], gi)
            sg = np.array([gs[n] for n in rec["frontier"].tolist()])
            assert np.max(np.abs(sg - rec["scores"])) <= P.SCORE_TOL
            kept = P.gpu_kept(tr[kv], gi)
            diff = np.array(sorted(set(kept.tolist()) ^ set(rec["kept"].tolist())), dtype=np.int64)
            _, bad = P.exempt_nodes(rec, sched[lv - 1], diff)
            assert not bad, f"level {lv} head {h}: unexplained set mismatch {bad[:5]}"
    t.close()


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("varying", [False, True])
def test_decode_end_to_end(name, varying):
    w, sched, K, V, trees, t, Kd, Vd = setup(name)
    g = w.group
    n = w.n_tokens
    for step in range(w.steps):
        if w.appends:
            t.append(Kd[:, n].contiguous(), Vd[:, n].contiguous())
            for h in range(w.num_kv_heads):
                zo.append_token(trees[h], K[h, n])
            n += 1
        # a context-dependent schedule: every level's p moves with the step
        s = [min(1.0, x + 0.02 * step) for x in sched] if varying else sched
        t.set_top_p_levels(s)
        q = gen.step_queries(w, step, n, gen.host_fetch(K))
        o = t.decode(P.upload(q, w))
        torch.cuda.synchronize()
        o = o.cpu().numpy()
        traces = {lv: t.trace(lv) for lv in range(0, w.levels + 1)}
        o_ref, routes = zo.decode(trees, V, q, s, w.keep_sink, return_routes=True)
        for h in range(w.num_q_heads):
            kv, gi = divmod(h, g)
            tr = {lv: traces[lv][kv] for lv in traces}
            rep = P.compare_route(routes[h], tr, gi, w.block, s)
            assert not rep["bad"], f"step {step} head {h}: {rep['bad'][:5]}"
            toks = P.gpu_tokens(tr[0], gi, w.block, n, w.keep_sink)
            e1 = P.out_err(o[h], zo.attend(K[kv][:n], V[kv][:n], q[h], toks))
            assert e1 <= P.OUT_RTOL, f"step {step} head {h}: attention over the GPU set err {e1:.3e}"
            if not rep["exempt"]:
                e2 = P.out_err(o[h], o_ref[h])
                assert e2 <= P.OUT_RTOL, f"step {step} head {h}: output err {e2:.3e}"
    # restoring the config's p: the next decode routes with it again
    t.set_top_p_levels(None)
    q = gen.step_queries(w, 50, n, gen.host_fetch(K))
    t.decode(P.upload(q, w))
    torch.cuda.synchronize()
    traces = {lv: t.trace(lv) for lv in range(0, w.levels + 1)}
    _, routes = zo.decode(trees, V, q, w.top_p, w.keep_sink, return_routes=True)
    for h in range(w.num_q_heads):
        kv, gi = divmod(h, g)
        rep = P.compare_route(routes[h], {lv: traces[lv][kv] for lv in traces}, gi, w.block, w.top_p)
        assert not rep["bad"], f"restored p, head {h}: {rep['bad'][:5]}"
    t.close()

