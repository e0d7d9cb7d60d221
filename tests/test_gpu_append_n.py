"""GPU parity of multi-token append (zha_tree_append_n) against the oracle.

A tree built over N0 tokens grows by chunks of m tokens (crossing key-tile, block and
upper-node boundaries, mixed with single-token appends); after every chunk its planes at
every level match an oracle tree built from scratch over the same tokens, the quantised
router copies match the oracle's quantisation, and decode agrees end to end.  Also: a
chunk that would pass the capacity is refused and leaves the tree as it was.
Tolerances: tests/parity.py (planes as in test_gpu_parity.py).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import parity as P
from oracle import zha_oracle as zo
from workloads import configs as wc, gen

pytestmark = pytest.mark.gpu

# (workload, N0, chunk sizes; 1 = a single-token append)
CASES = {
    # tiles of 128 tokens, level-6 nodes of 4,096: 100 crosses a tile, 3000 a level-6 node
    "deep_small": (wc.DEEP, 16_384 + 37, [100, 1, 3000, 1, 7]),
    "tiny": (wc.TINY, 1000, [3, 64, 1, 500]),
    "ultra_small": (wc.ULTRA, 70_001, [511, 1, 4096]),
    "deep_fp4": (wc.DEEP.with_(planes="fp4"), 16_384 + 37, [100, 1, 3000]),
    "light_bf16": (wc.light(32_768).with_(planes="bf16"), 32_768 - 5, [700, 1, 9]),
}


def check_planes(w, t, trees):
    for lv in range(1, w.levels + 1):
        s, cc = t.level(lv)
        s, cc = s.cpu().numpy(), cc.cpu().numpy()
        for h in range(w.num_kv_heads):
            so, co = trees[h].levels[lv - 1]
            assert s[h].shape == so.shape, f"level {lv}: {s[h].shape} nodes vs {so.shape}"
            es = np.max(np.abs(s[h] - so)) / max(1.0, np.max(np.abs(so)))
            ec = np.max(np.abs(cc[h] - co))
            assert es < 1e-4 and ec < 1e-3, f"level {lv} head {h}: s err {es:.2e}, c err {ec:.2e}"
        if w.planes != "f32" and lv in P.router_levels(w):
            rp = t.router_planes(lv)
            sq = (P.decode_fp4(rp[0].cpu().numpy(), rp[1].cpu().numpy()) if w.planes == "fp4"
                  else rp.float().cpu().numpy().astype(np.float64))
            for h in range(w.num_kv_heads):
                lo, hi = P.quant_bounds(w.planes, trees[h].levels[lv - 1][0])
                assert np.all((sq[h] >= lo) & (sq[h] <= hi)), f"level {lv} head {h}: router copy off bounds"


@pytest.mark.parametrize("name", list(CASES))
def test_append_n_matches_rebuild(name):
    base, n0, chunks = CASES[name]
    total = n0 + sum(chunks)
    w = base.with_(n_tokens=n0, steps=total - n0, appends=True)
    K, V, refs = P.host_inputs(w)
    t = P.make_tree(w, capacity=total)
    Kd, Vd = P.upload(K, w), P.upload(V, w)
    t.build(Kd, Vd, n0, P.upload(refs, w))
    # chunks come from separate buffers (as a caller would pass them); the cache rows past
    # N0 start zeroed, so every appended row must be copied in
    Kn, Vn = Kd.clone(), Vd.clone()
    Kd[:, n0:] = 0
    Vd[:, n0:] = 0
    n = n0
    for m in chunks:
        if m == 1:
            t.append(Kn[:, n].contiguous(), Vn[:, n].contiguous())
        else:
            t.append_n(Kn[:, n:n + m].contiguous(), Vn[:, n:n + m].contiguous())
        n += m
        assert t.n_tokens == n
        torch.cuda.synchronize()
        trees = [zo.build_tree(K[h], refs[h], w.block, w.levels, n) for h in range(w.num_kv_heads)]
        check_planes(w, t, trees)
    # decode end to end on the grown tree
    g = w.group
    q = gen.step_queries(w, 7, n, gen.host_fetch(K))
    o = t.decode(P.upload(q, w)).cpu().numpy()
    traces = {lv: t.trace(lv) for lv in range(0, w.levels + 1)}
    keys = t.route_mode == 2   # every level scored from the keys: no plane copy is read
    tol_fn = lambda kv, qh: (lambda lv, fr: P.SCORE_TOL + P.flip_allowance(w, trees[kv], lv, fr, qh, keys))
    reps = P.check_decode(P.router_trees(w, trees, keys), K, V, q, o, traces, w.top_p, w.keep_sink, n,
                          tol_fn=tol_fn)
    P.assert_exemption_rates(f"{name} after appends", reps)
    t.close()


def test_append_n_capacity():
    from hierarchical_tree_indexed_03_amd import zha
    w = wc.TINY.with_(n_tokens=100, steps=10, appends=True)
    K, V, refs = P.host_inputs(w)
    t = P.make_tree(w, capacity=110)
    Kd, Vd = P.upload(K, w), P.upload(V, w)
    t.build(Kd, Vd, 100, P.upload(refs, w))
    too_many = torch.zeros(1, 11, w.head_dim, dtype=Kd.dtype, device="cuda")
    with pytest.raises(zha.ZhaError) as e:
        t.append_n(too_many, too_many)
    assert e.value.status == 3
    assert t.n_tokens == 100
    Kn, Vn = Kd.clone(), Vd.clone()
    Kd[:, 100:] = 0
    Vd[:, 100:] = 0
    t.append_n(Kn[:, 100:110].contiguous(), Vn[:, 100:110].contiguous())
    assert t.n_tokens == 110
    torch.cuda.synchronize()
    check_planes(w, t, [zo.build_tree(K[0], refs[0], w.block, w.levels, 110)])
    t.close()


@pytest.mark.parametrize("name", ["deep_small", "tiny", "ultra_small"])
def test_prefill_equals_append_then_decode(name):
    """zha_prefill over a chunk = one zha_tree_append + zha_decode per token (bitwise: the
    same kernels in the same order), and the last query matches the oracle end to end."""
    base, n0, _ = CASES[name]
    m = 24
    w = base.with_(n_tokens=n0, steps=m, appends=True)
    K, V, refs = P.host_inputs(w)
    Kd, Vd = P.upload(K, w), P.upload(V, w)
    Rd = P.upload(refs, w)
    qs = np.stack([gen.step_queries(w, i, n0 + i + 1, gen.host_fetch(K)) for i in range(m)])
    Qd = P.upload(qs, w)
    kc, vc = Kd[:, n0:n0 + m].contiguous(), Vd[:, n0:n0 + m].contiguous()
    # chunked prefill on one tree ...
    t1 = P.make_tree(w, capacity=n0 + m)
    t1.build(Kd, Vd, n0, Rd)
    out1 = t1.prefill(kc, vc, Qd).cpu().numpy()
    assert t1.n_tokens == n0 + m
    traces = {lv: t1.trace(lv) for lv in range(0, w.levels + 1)}
    # ... and token by token on another
    t2 = P.make_tree(w, capacity=n0 + m)
    t2.build(Kd, Vd, n0, Rd)
    out2 = np.empty_like(out1)
    for i in range(m):
        t2.append(kc[:, i].contiguous(), vc[:, i].contiguous())
        out2[i] = t2.decode(Qd[i].contiguous()).cpu().numpy()
    assert np.array_equal(out1, out2), "prefill differs from append + decode"
    # the last query against the oracle, with its routing trace
    n = n0 + m
    trees = [zo.build_tree(K[h], refs[h], w.block, w.levels, n) for h in range(w.num_kv_heads)]
    reps = P.check_decode(trees, K, V, qs[-1], out1[-1], traces, w.top_p, w.keep_sink, n, label="last query")
    P.assert_exemption_rates(f"{name} prefill last query", reps)
    # a chunk past the capacity is refused before anything is enqueued
    from hierarchical_tree_indexed_03_amd import zha
    with pytest.raises(zha.ZhaError) as e:
        t1.prefill(kc[:, :1].contiguous(), vc[:, :1].contiguous(), Qd[:1].contiguous())
    assert e.value.status == 3 and t1.n_tokens == n
    t1.close()
    t2.close()
