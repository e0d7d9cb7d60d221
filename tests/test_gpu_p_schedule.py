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


@pytest.mark.parametrize("path", [0, 1], ids=["decode_path", "list_path"])
@pytest.mark.parametrize("name", list(CASES))
def test_teacher_forced_sets(name, path):
    w, sched, K, V, trees, t, _, _ = setup(name)
    q = gen.step_queries(w, 100, w.n_tokens, gen.host_fetch(K))
    rep = P.teacher_forced(t, trees, q, P.upload(q, w), sched, w.keep_sink, path)
    assert not rep["bad"], f"{rep['bad'][:5]}"
    assert rep["max_err"] <= P.SCORE_TOL
    P.assert_exemption_rates(f"{name} teacher-forced path {path}", rep)
    t.close()


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("varying", [False, True])
def test_decode_end_to_end(name, varying):
    w, sched, K, V, trees, t, Kd, Vd = setup(name)
    n = w.n_tokens
    reps = []
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
        reps += P.check_decode(trees, K, V, q, o, traces, s, w.keep_sink, n, label=f"step {step}")
    # restoring the config's p: the next decode routes with it again
    t.set_top_p_levels(None)
    q = gen.step_queries(w, 50, n, gen.host_fetch(K))
    o = t.decode(P.upload(q, w))
    torch.cuda.synchronize()
    o = o.cpu().numpy()
    traces = {lv: t.trace(lv) for lv in range(0, w.levels + 1)}
    reps += P.check_decode(trees, K, V, q, o, traces, w.top_p, w.keep_sink, n, label="restored p")
    P.assert_exemption_rates(f"{name} end to end", reps)
    t.close()
