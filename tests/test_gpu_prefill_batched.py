"""GPU parity of the batched causal prefill (zha_prefill_batched) against the oracle.

Query i of a chunk routes over the tree of the tokens up to and including its own (blog
"Zyphra Hierarchical Attention", section "Routing through the tree"), so the oracle for it
is a tree built from scratch over those tokens and the plain decode on it.  For every
query of every sub-batch (each traced after its call) and every query head:
  * every node of the query's tree scores within 1e-4 of the oracle's score at every
    level, the rightmost node included (the query's own partial version of it), and the
    nodes right of it score -inf;
  * the kept set at every level is the oracle's top-p of the GPU's frontier (the mass band
    and verified near-tie swaps only, at the stated rates), tests/parity.py;
  * the output matches attention over the kept blocks' tokens up to the query's own (and
    the sink), and the oracle's own decode whenever no exemption was used.
One call over the whole chunk must give the same bits as the sub-batches one call each.
The chunks cross blocks, key tiles and upper nodes, end ragged (m not a multiple of the
batch), start at one token, and the batch runs from 1 to the chunk.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import parity as P
from oracle import zha_oracle as zo
from workloads import configs as wc, gen

pytestmark = pytest.mark.gpu

# (workload, tokens before the chunk, chunk length, queries per sub-batch)
CASES = {
    "tiny": (wc.TINY, 1000, 37, 16),
    "tiny_from_one": (wc.TINY, 1, 21, 5),
    "tiny_batch1": (wc.TINY, 4093, 3, 1),
    "deep_small": (wc.DEEP, 16_384 + 37, 24, 16),
    # level 1 of 16K nodes nearly all in each head's frontier: past the LDS list, the level
    # is read whole with the parents' kept bitmap in LDS
    "deep_scan": (wc.DEEP, 65_536 + 100, 6, 6),
    # more than 65,536 level-1 nodes: the kept bitmap is built in global memory, by words
    # (a scanned level) and node by node (a listed one)
    "deep_scan_wide": (wc.DEEP, 270_000, 3, 3),
    "ultra_list_wide": (wc.ULTRA, 720_901, 4, 4),
    "ultra_small": (wc.ULTRA, 70_001, 20, 8),
    "wide_small": (wc.WIDE, 5_000, 20, 7),
    "light_bf16": (wc.light(32_768).with_(planes="bf16"), 32_768 - 5, 30, 30),
}


def setup(w, n0, m):
    K, V, refs = P.host_inputs(w)
    Kd, Vd, Rd = P.upload(K, w), P.upload(V, w), P.upload(refs, w)
    qs = np.stack([gen.step_queries(w, i, n0 + i + 1, gen.host_fetch(K)) for i in range(m)])
    # copies (a slice of a one-head cache is contiguous already and would see the zeroing)
    kc, vc = Kd[:, n0:n0 + m].clone(), Vd[:, n0:n0 + m].clone()
    # the cache rows past n0 start zeroed: prefill must copy every chunk row in
    Kd[:, n0:] = 0
    Vd[:, n0:] = 0
    return K, V, refs, Kd, Vd, Rd, qs, kc, vc


@pytest.mark.parametrize("name", list(CASES))
def test_prefill_batched_matches_oracle(name):
    base, n0, m, batch = CASES[name]
    w = base.with_(n_tokens=n0, steps=m, appends=True)
    K, V, refs, Kd, Vd, Rd, qs, kc, vc = setup(w, n0, m)
    Qd = P.upload(qs, w)
    g, L, b = w.group, w.levels, w.block
    print(f"[prefill] {name}: n0={n0} m={m} batch={batch}", flush=True)
    # sub-batch by sub-batch, each traced and checked against the oracle
    t = P.make_tree(w, capacity=n0 + m)
    t.build(Kd.clone(), Vd.clone(), n0, Rd)
    out = np.empty((m, w.num_q_heads, w.head_dim), np.float32)
    reps = []
    for s0 in range(0, m, batch):
        mb = min(batch, m - s0)
        o = t.prefill_batched(kc[:, s0:s0 + mb].contiguous(), vc[:, s0:s0 + mb].contiguous(),
                              Qd[s0:s0 + mb].contiguous(), batch)
        out[s0:s0 + mb] = o.cpu().numpy()
        assert t.n_tokens == n0 + s0 + mb
        tr = {}
        for lv in range(1, L + 1):
            sc, kb, own, mb_t, n_end = t.prefill_trace(lv)
            assert (mb_t, n_end) == (mb, n0 + s0 + mb)
            tr[lv] = (sc.numpy(), kb.numpy(), -(-n_end // b ** lv), own.numpy())
        for i in range(mb):
            qi = s0 + i
            n_i = n0 + qi + 1
            trees = P.oracle_trees(w, K, refs, n_i)
            # the query's own rightmost node of every level: the oracle's node over [0, n_i)
            for lv in tr:
                nd = (n_i - 1) // b ** lv
                for kv in range(w.num_kv_heads):
                    so, co = trees[kv].levels[lv - 1]
                    x = tr[lv][3][kv, i].astype(np.float64)
                    es = np.max(np.abs(x[:, :-2] - so[nd])) / max(1.0, np.max(np.abs(so[nd])))
                    ec = np.max(np.abs(x[:, -2] - co[nd]))
                    assert es < 1e-4 and ec < 1e-3, \
                        f"{name} query {qi} level {lv} KV head {kv}: own node s err {es:.2e}, c err {ec:.2e}"
            for h in range(w.num_q_heads):
                kv, gi = divmod(h, g)
                pair = i * g + gi
                scores = {lv: tr[lv][0][kv, pair] for lv in tr}
                kept = {lv: P.kept_from_bits(tr[lv][1][kv, pair], tr[lv][2]) for lv in tr}
                rep, blocks = P.compare_prefill_pair(trees[kv], qs[qi][h], scores, kept, w.top_p)
                assert not rep["bad"], f"{name} query {qi} head {h}: {rep['bad'][:4]}"
                tok = (blocks[:, None] * b + np.arange(b)[None, :]).ravel()
                tok = tok[tok < n_i]
                if w.keep_sink:
                    tok = np.union1d([0], tok)
                e1 = P.out_err(out[qi, h], zo.attend(K[kv][:n_i], V[kv][:n_i], qs[qi][h], tok))
                assert e1 <= P.OUT_RTOL, f"{name} query {qi} head {h}: attention over the kept set, error {e1:.3e}"
                if rep["same"]:
                    r = zo.route(trees[kv], qs[qi][h], w.top_p, w.keep_sink)
                    assert np.array_equal(r["blocks"], blocks), f"{name} query {qi} head {h}: blocks differ"
                    e2 = P.out_err(out[qi, h], zo.attend(K[kv][:n_i], V[kv][:n_i], qs[qi][h], r["tokens"]))
                    assert e2 <= P.OUT_RTOL, f"{name} query {qi} head {h}: output error {e2:.3e}"
                reps.append(rep)
    P.assert_exemption_rates(f"{name} batched prefill", reps)
    # the whole chunk in one call: the same bits
    t2 = P.make_tree(w, capacity=n0 + m)
    t2.build(Kd.clone(), Vd.clone(), n0, Rd)
    o2 = t2.prefill_batched(kc, vc, Qd, batch).cpu().numpy()
    assert t2.n_tokens == n0 + m
    assert np.array_equal(o2, out), "one call differs from its sub-batches called one by one"
    t.close()
    t2.close()


def test_prefill_batched_errors():
    from hierarchical_tree_indexed_03_amd import zha
    w = wc.TINY.with_(n_tokens=100, steps=10, appends=True)
    K, V, refs, Kd, Vd, Rd, qs, kc, vc = setup(w, 100, 10)
    Qd = P.upload(qs, w)
    t = P.make_tree(w, capacity=109)
    t.build(Kd, Vd, 100, Rd)
    with pytest.raises(zha.ZhaError) as e:       # past the capacity: nothing enqueued
        t.prefill_batched(kc, vc, Qd, 4)
    assert e.value.status == 3 and t.n_tokens == 100
    with pytest.raises(ValueError):              # batch outside 1..128
        t.prefill_batched(kc, vc, Qd, 129)
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    out = torch.empty(10, w.num_q_heads, w.head_dim, dtype=torch.float32, device="cuda")
    with pytest.raises(zha.ZhaError) as e:       # workspace too small
        zha.zha_prefill_batched(t.handle, kc[:, :9].contiguous(), vc[:, :9].contiguous(), Qd, out, 9, 4, ws, 16)
    assert e.value.status == 4 and t.n_tokens == 100
    t.close()
