"""GPU parity of quantised router planes (zha_config.plane_dtype bf16 and MX FP4) against
the oracle.

The oracle routes over its planes with s quantised (bf16, or OCP MX FP4 with a scale per
32 elements) at every level the router reads planes at (all but a key-form level 1);
offsets stay full precision.  Checked here, for both formats:

* the quantiser, element by element: the GPU's fp32 s lies within S_BAND of the oracle's
  fp64 s, and the GPU's quantised copy equals the oracle's quantisation of s wherever the
  bounds [lo, hi] of tests/parity.py coincide (else it lies between them);
* teacher-forced scores on the oracle's frontiers, within SCORE_TOL plus each node's
  rounding-flip allowance, and the kept sets (tests/parity.py rules);
* decode end to end after appends (the append refreshes the bf16 copies).

Geometries: f32 queries (fp32 MFMA on widened planes; R 4 and R 16), the deep tree (key-form level 1,
bf16 planes above it, selected top-down), one 256-key level (R 16), the light router
(R 1) top-down and through the large-level path, and the 16M geometry at a small size.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import parity as P
from oracle import zha_oracle as zo
from workloads import configs as wc, gen

pytestmark = pytest.mark.gpu

GEOMS = {
    "tiny": wc.TINY,
    "tiny_r16": wc.TINY.with_(num_ref=16),
    "deep_small": wc.DEEP.with_(n_tokens=16_384 + 37, steps=2),
    "wide_small": wc.WIDE.with_(n_tokens=8_192 + 100, steps=2),
    "light_small": wc.light(32_768, steps=2).with_(n_tokens=32_768 - 5),
    # level 1 holds 36,001 nodes: scored from the union list, selected by the large-level path
    "light_general": wc.light(288_003, steps=1).with_(num_kv_heads=1, num_q_heads=8),
    "ultra_small": wc.ULTRA.with_(n_tokens=70_001, steps=2),
    # head_dim 64 with bf16 keys: the narrow build and the scorers at d = 64
    "light_d64": wc.light(32_768, steps=2).with_(n_tokens=20_000 + 3, head_dim=64),
    # R 4, b 4 at d = 64: narrow build with key-form token weights, key-form level 1
    "deep_d64_r4": wc.DEEP.with_(n_tokens=10_000 + 3, head_dim=64, num_ref=4, levels=4, steps=2),
}
SMALL = {f"{fmt}-{name}": w.with_(planes=fmt) for fmt in ("bf16", "fp4") for name, w in GEOMS.items()}


class Case:
    def __init__(self, w: wc.Workload):
        self.w = w
        self.p = w.top_p
        self.K, self.V, self.refs = P.host_inputs(w)
        self.trees = P.oracle_trees(w, self.K, self.refs, w.n_tokens)
        self.t = P.make_tree(w)
        self.t.set_route_mode(1)   # the union frontiers, which read the quantised plane copies
        self.Kd, self.Vd = P.upload(self.K, w), P.upload(self.V, w)
        self.t.build(self.Kd, self.Vd, w.n_tokens, P.upload(self.refs, w))
        self.n = w.n_tokens

    def append(self):
        w, n = self.w, self.n
        self.t.append(self.Kd[:, n].contiguous(), self.Vd[:, n].contiguous())
        for h in range(w.num_kv_heads):
            zo.append_token(self.trees[h], self.K[h, n])
        self.n += 1

    def queries(self, step):
        return gen.step_queries(self.w, step, self.n, gen.host_fetch(self.K))

    def tol_fn(self, kv, q):
        tree = self.trees[kv]
        return lambda lv, fr: P.SCORE_TOL + P.flip_allowance(self.w, tree, lv, fr, q)


_CACHE = {}


def case(name) -> Case:
    if name not in _CACHE:
        _CACHE.clear()
        _CACHE[name] = Case(SMALL[name])
    return _CACHE[name]


def check_quantiser(c: Case):
    w = c.w
    for lv in range(1, w.levels + 1):
        if lv not in P.router_levels(w):
            from hierarchical_tree_indexed_03_amd import zha
            with pytest.raises(zha.ZhaError):
                c.t.router_planes(lv)
            continue
        s32 = c.t.level(lv)[0].cpu().numpy().astype(np.float64)
        rp = c.t.router_planes(lv)
        if w.planes == "fp4":
            sq = P.decode_fp4(rp[0].cpu().numpy(), rp[1].cpu().numpy())
        else:
            sq = rp.float().cpu().numpy().astype(np.float64)
        for h in range(w.num_kv_heads):
            so = c.trees[h].levels[lv - 1][0]
            err = float(np.max(np.abs(s32[h] - so)))
            assert err <= P.S_BAND, f"level {lv} head {h}: fp32 s differs from the oracle by {err:.2e}"
            lo, hi = P.quant_bounds(w.planes, so)
            mid = zo.QUANTISERS[w.planes](so)
            sure = lo == hi
            assert np.array_equal(sq[h][sure], mid[sure]), f"level {lv} head {h}: bf16 copy differs"
            # quantisation is monotone for a fixed scale: s_gpu within S_BAND of s lands in [lo, hi]
            assert np.all((sq[h] >= lo) & (sq[h] <= hi)), f"level {lv} head {h}: bf16 copy outside [lo, hi]"


@pytest.mark.parametrize("name", list(SMALL))
def test_router_planes_quantiser(name):
    check_quantiser(case(name))


@pytest.mark.parametrize("path", [0, 1], ids=["decode_path", "list_path"])
@pytest.mark.parametrize("name", list(SMALL))
def test_teacher_forced_scores_and_sets(name, path):
    c = case(name)
    w = c.w
    q = c.queries(100)
    rep = P.teacher_forced(c.t, P.router_trees(w, c.trees), q, P.upload(q, w), c.p, w.keep_sink, path,
                           tol_fn=c.tol_fn)
    assert not rep["bad"], f"{rep['bad'][:5]}"
    P.assert_exemption_rates(f"{name} teacher-forced path {path}", rep)


@pytest.mark.parametrize("name", list(SMALL))
def test_decode_end_to_end(name):
    c = case(name)
    w = c.w
    reps = []
    for step in range(max(1, w.steps)):
        if w.appends and w.steps:
            c.append()
        q = c.queries(step)
        o = c.t.decode(P.upload(q, w))
        torch.cuda.synchronize()
        o = o.cpu().numpy()
        traces = {lv: c.t.trace(lv) for lv in range(0, w.levels + 1)}
        reps += P.check_decode(P.router_trees(w, c.trees), c.K, c.V, q, o, traces, c.p, w.keep_sink, c.n,
                               tol_fn=c.tol_fn, label=f"step {step}")
    P.assert_exemption_rates(f"{name} end to end", reps)
    # the appended rows' bf16 copies follow the refreshed planes
    check_quantiser(c)
