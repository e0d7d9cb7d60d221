"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on seeded inputs.

Shapes: the tiny workload in full, and the deep / wide / light / ultra geometries at token
counts the oracle finishes in seconds (several tiles, ragged tails), each over a few decode
steps that append one token first.  Tolerances are those of tests/parity.py.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import parity as P
from oracle import zha_oracle as zo
from workloads import configs as wc, gen

pytestmark = pytest.mark.gpu

SMALL = {
    "tiny": wc.TINY,
    "deep_small": wc.DEEP.with_(n_tokens=16_384 + 37, steps=3),
    "wide_small": wc.WIDE.with_(n_tokens=8_192 + 100, steps=3),
    "light_small": wc.light(32_768, steps=3).with_(n_tokens=32_768 - 5),
    "ultra_small": wc.ULTRA.with_(n_tokens=70_001, steps=2),
    "light_d64": wc.light(32_768, steps=2).with_(n_tokens=20_000 + 3, head_dim=64),
    "deep_d64_r4": wc.DEEP.with_(n_tokens=10_000 + 3, head_dim=64, num_ref=4, levels=4, steps=2),
    # one or two (node, plane) pairs per build tile: each pair's log-sum-exp split over 64 lanes
    "wide_r1": wc.WIDE.with_(n_tokens=6_144 + 77, num_ref=1, steps=2),
    "b128_r2_f32": wc.WIDE.with_(block=128, levels=2, num_ref=2, dtype="f32", n_tokens=20_000 + 9, steps=2),
    # key-form level 1 at every block size it takes (8, 2 and 1 nodes per 16-token tile)
    "keys_b2": wc.DEEP.with_(block=2, levels=8, n_tokens=12_000 + 7, steps=2),
    "keys_b8": wc.DEEP.with_(block=8, levels=4, n_tokens=16_384 + 19, steps=2),
    "keys_b16": wc.DEEP.with_(block=16, levels=3, n_tokens=20_000 + 3, steps=2),
    "keys_b2_r2_d64": wc.DEEP.with_(block=2, num_ref=2, head_dim=64, levels=8, n_tokens=9_000 + 1, steps=2),
    # the deep geometries again with the per-level union frontiers (their default scores every
    # level from the keys)
    "deep_small_frontier": wc.DEEP.with_(n_tokens=16_384 + 37, steps=3),
    "deep_d64_r4_frontier": wc.DEEP.with_(n_tokens=10_000 + 3, head_dim=64, num_ref=4, levels=4, steps=2),
    # every level from the keys with a top level above level 4 of more than one node and a
    # ragged tail at every level; one with exactly four levels (no level derived above 4)
    "keys_all_l7": wc.DEEP.with_(levels=7, n_tokens=40_000 + 13, steps=2),
    "keys_all_r8_l4": wc.DEEP.with_(num_ref=8, levels=4, n_tokens=5_000 + 1, steps=2),
}
# route mode per case (0: the config's default; 1: union frontiers; 2: every level from the keys)
ROUTE = {"deep_small_frontier": 1, "deep_d64_r4_frontier": 1}


class Case:
    def __init__(self, w: wc.Workload, top_p=None, route=0):
        self.w = w
        self.p = w.top_p if top_p is None else top_p
        self.K, self.V, self.refs = P.host_inputs(w)
        self.trees = P.oracle_trees(w, self.K, self.refs, w.n_tokens)
        self.t = P.make_tree(w, top_p=self.p)
        self.t.set_route_mode(route)
        self.Kd, self.Vd, self.Rd = P.upload(self.K, w), P.upload(self.V, w), P.upload(self.refs, w)
        self.t.build(self.Kd, self.Vd, w.n_tokens, self.Rd)
        self.n = w.n_tokens

    def append(self):
        w, n = self.w, self.n
        self.t.append(self.Kd[:, n].contiguous(), self.Vd[:, n].contiguous())
        for h in range(w.num_kv_heads):
            zo.append_token(self.trees[h], self.K[h, n])
        self.n += 1

    def queries(self, step):
        return gen.step_queries(self.w, step, self.n, gen.host_fetch(self.K))

    def decode(self, q):
        qd = P.upload(q, self.w)
        o = self.t.decode(qd)
        torch.cuda.synchronize()
        traces = {lv: self.t.trace(lv) for lv in range(0, self.w.levels + 1)}
        return o.cpu().numpy(), traces


_CACHE = {}


def case(name) -> Case:
    if name not in _CACHE:
        _CACHE.clear()
        _CACHE[name] = Case(SMALL[name], route=ROUTE.get(name, 0))
    return _CACHE[name]


# the scoring each case's decode runs: every level from the keys on the block-4 key-form
# geometries unless the case asks for the union frontiers
ROUTE_EXPECT = {"deep_small": 2, "deep_d64_r4": 2, "keys_all_l7": 2, "keys_all_r8_l4": 2,
                "deep_small_frontier": 1, "deep_d64_r4_frontier": 1, "keys_b2": 1, "wide_small": 1}


@pytest.mark.parametrize("name", list(ROUTE_EXPECT))
def test_route_mode_in_use(name):
    assert case(name).t.route_mode == ROUTE_EXPECT[name]


@pytest.mark.parametrize("name", list(SMALL))
def test_planes_match_oracle(name):
    c = case(name)
    w = c.w
    for lv in range(1, w.levels + 1):
        s, cc = c.t.level(lv)
        s, cc = s.cpu().numpy(), cc.cpu().numpy()
        for h in range(w.num_kv_heads):
            so, co = c.trees[h].levels[lv - 1]
            es = np.max(np.abs(s[h] - so)) / max(1.0, np.max(np.abs(so)))
            ec = np.max(np.abs(cc[h] - co))
            assert es < 1e-4 and ec < 1e-3, f"level {lv} head {h}: s err {es:.2e}, c err {ec:.2e}"


@pytest.mark.parametrize("path", [0, 1], ids=["decode_path", "list_path"])
@pytest.mark.parametrize("name", list(SMALL))
def test_teacher_forced_scores_and_sets(name, path):
    """Every level routed from the oracle's own frontier: path 0 runs the kernels the
    decode runs at that level (dense scoring and top-down selection on the top levels),
    path 1 the large-level kernels."""
    c = case(name)
    w = c.w
    q = c.queries(100)
    rep = P.teacher_forced(c.t, c.trees, q, P.upload(q, w), c.p, w.keep_sink, path)
    assert not rep["bad"], f"{rep['bad'][:5]}"
    assert rep["max_err"] <= P.SCORE_TOL, f"max score error {rep['max_err']:.3e}"
    P.assert_exemption_rates(f"{name} teacher-forced path {path}", rep)


@pytest.mark.parametrize("name", list(SMALL))
def test_decode_end_to_end(name):
    c = case(name)
    w = c.w
    reps = []
    for step in range(w.steps if w.steps else 1):
        if w.appends:
            c.append()
        q = c.queries(step)
        o, traces = c.decode(q)
        reps += P.check_decode(c.trees, c.K, c.V, q, o, traces, c.p, w.keep_sink, c.n, label=f"step {step}")
    P.assert_exemption_rates(f"{name} end to end", reps)


@pytest.mark.parametrize("name", ["tiny", "deep_small", "wide_small"])
def test_dense_decode(name):
    c = case(name)
    q = c.queries(7)
    o = c.t.decode_dense(P.upload(q, c.w)).cpu().numpy()
    ref = zo.dense_decode(c.K, c.V, q, c.n)
    assert P.out_err(o, ref) <= P.OUT_RTOL


@pytest.mark.parametrize("name", ["tiny", "deep_small", "light_small"])
def test_p1_is_dense(name):
    w = SMALL[name]
    c = Case(w.with_(steps=0), top_p=1.0)
    q = c.queries(3)
    qd = P.upload(q, w)
    o = c.t.decode(qd).cpu().numpy()
    od = c.t.decode_dense(qd).cpu().numpy()
    ref = zo.dense_decode(c.K, c.V, q, c.n)
    assert P.out_err(o, ref) <= P.OUT_RTOL
    assert P.out_err(o, od) <= 1e-4
    tr0 = c.t.trace(0)
    for kv in range(w.num_kv_heads):
        assert len(tr0[kv]["nodes"]) == w.nodes(1, c.n)


def test_deterministic():
    c = case("deep_small")
    q = c.queries(11)
    o1, t1 = c.decode(q)
    o2, t2 = c.decode(q)
    assert np.array_equal(o1, o2)
    for lv in t1:
        for a, b in zip(t1[lv], t2[lv]):
            assert torch.equal(a["nodes"], b["nodes"]) and torch.equal(a["masks"], b["masks"])
            if a["keep"] is not None:
                assert torch.equal(a["keep"], b["keep"])


def test_append_equals_rebuild():
    w = SMALL["deep_small"].with_(steps=70)
    c = Case(w)
    for _ in range(70):
        c.append()
    t2 = P.make_tree(w)
    t2.build(c.Kd, c.Vd, c.n, c.Rd)
    for lv in range(1, w.levels + 1):
        s1, c1 = c.t.level(lv)
        s2, c2 = t2.level(lv)
        assert torch.allclose(s1, s2, atol=1e-4, rtol=1e-4), f"level {lv} s"
        assert torch.allclose(c1, c2, atol=1e-3, rtol=1e-4), f"level {lv} c"
