"""GPU parity of the reference-query fit (zha_fit_step) against the oracle.

One step with lr = 0 on seeded inputs: the loss of every KV head (KL of the dense node mass
to the router's probabilities, summed over levels, averaged over the group's training
queries) and its gradient in the reference queries, against oracle.fit_grad on the same
values (keys and queries as stored, reference queries rounded to the cache dtype as the
library does).  Tolerances: the loss within 2e-4 per level (score and log-mass errors of
about 1e-4 each) plus 1e-5 relative; the gradient within 2e-3 of its largest element plus
the arg-max flip allowance of tests/parity.py (pairs of planes within 2e-4 of each other).
Then the update itself (refs -= lr * grad in float32) and a short descent: ten steps with a
fixed lr lower the loss of every head.
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
    # name: (workload, training queries per head (nq))
    "tiny_f32": (wc.TINY.with_(n_tokens=1000), 4),
    "d64_r2_bf16": (wc.TINY.with_(num_ref=2, dtype="bf16", n_tokens=3001, block=8, levels=3), 4),
    "deep_small": (wc.DEEP.with_(n_tokens=4096 + 37, levels=4), 1),
    "light_small": (wc.light(32_768).with_(n_tokens=9000), 2),
    # 80 training queries per KV head: two LDS query blocks in the scoring, two per lane in
    # the per-node sums
    "deep_q80": (wc.DEEP.with_(n_tokens=2048 + 5, levels=3, num_kv_heads=1, num_q_heads=8), 10),
}


def inputs(w, nq, seed=5):
    K, V, refs = P.host_inputs(w)
    rng = np.random.default_rng(seed)
    refs32 = (refs + 0.01 * rng.standard_normal(refs.shape)).astype(np.float32)
    qs = np.stack([gen.step_queries(w, s, w.n_tokens, gen.host_fetch(K)) for s in range(nq)])
    return K, V, refs32, qs


def oracle_refs(w, refs32):
    r = refs32.astype(np.float64)
    return zo.bf16_round(r) if w.dtype == "bf16" else r


def group_queries(w, qs, kv):
    g = w.group
    return qs[:, kv * g:(kv + 1) * g, :].reshape(-1, w.head_dim).astype(np.float64)


@pytest.mark.parametrize("name", list(GEOMS))
def test_fit_loss_and_gradient(name):
    w, nq = GEOMS[name]
    n = w.n_tokens
    K, V, refs32, qs = inputs(w, nq)
    t = P.make_tree(w)
    Kd, Vd = P.upload(K, w), P.upload(V, w)
    rt = torch.from_numpy(refs32).cuda()
    loss, grad = t.fit_step(Kd, Vd, n, rt, P.upload(qs, w), lr=0.0)
    loss, grad = loss.cpu().numpy(), grad.cpu().numpy()
    assert np.array_equal(rt.cpu().numpy(), refs32), "lr = 0 changed the reference queries"
    ro = oracle_refs(w, refs32)
    for kv in range(w.num_kv_heads):
        qg = group_queries(w, qs, kv)
        lo, go = zo.fit_grad(K[kv], ro[kv], w.block, w.levels, n, qg)
        assert abs(loss[kv] - lo) <= 2e-4 * w.levels + 1e-5 * abs(lo), f"head {kv}: loss {loss[kv]:.6f} vs {lo:.6f}"
        allow = P.fit_flip_allowance(K[kv], ro[kv], w.block, w.levels, n, qg)
        err = np.abs(grad[kv] - go)
        tol = 2e-3 * np.max(np.abs(go)) + allow
        worst = np.unravel_index(np.argmax(err - tol), err.shape)
        assert np.all(err <= tol), (f"head {kv}: gradient [{worst}] {grad[kv][worst]:.6e} vs {go[worst]:.6e} "
                                    f"(largest {np.max(np.abs(go)):.3e}, allowance {allow[worst]:.2e})")
    t.close()


def test_fit_update_and_descent():
    w, nq = GEOMS["deep_small"]
    n = w.n_tokens
    K, V, refs32, qs = inputs(w, nq)
    t = P.make_tree(w)
    Kd, Vd = P.upload(K, w), P.upload(V, w)
    Qd = P.upload(qs, w)
    rt = torch.from_numpy(refs32).cuda()
    lr = 0.5
    before = rt.clone()
    l0, g0 = t.fit_step(Kd, Vd, n, rt, Qd, lr=lr)
    want = before - lr * g0
    assert torch.allclose(rt, want, rtol=1e-6, atol=1e-7), "refs != refs - lr * grad"
    losses = [l0.cpu().numpy()]
    for _ in range(9):
        li, _ = t.fit_step(Kd, Vd, n, rt, Qd, lr=lr, grad=False)
        losses.append(li.cpu().numpy())
    losses = np.array(losses)
    assert np.all(losses[-1] < losses[0]), f"loss did not fall: {losses[0]} -> {losses[-1]}"
    t.close()


def test_fit_argument_errors():
    from hierarchical_tree_indexed_03_amd import zha
    w, nq = GEOMS["tiny_f32"]
    K, V, refs32, qs = inputs(w, nq)
    t = P.make_tree(w)
    Kd, Vd = P.upload(K, w), P.upload(V, w)
    rt = torch.from_numpy(refs32).cuda()
    Qd = P.upload(qs, w)
    need = zha.zha_fit_workspace_bytes(t.cfg, w.n_tokens, nq)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    loss = torch.empty(1, device="cuda")
    with pytest.raises(zha.ZhaError) as e:
        zha.zha_fit_step(t.handle, Kd, Vd, w.capacity + 1, rt, Qd, nq, 0.0, loss, None, ws, need)
    assert e.value.status == 3
    with pytest.raises(zha.ZhaError) as e:
        zha.zha_fit_step(t.handle, Kd, Vd, w.n_tokens, rt, Qd, nq, 0.0, loss, None, ws, need - 256)
    assert e.value.status == 4
    assert zha.zha_fit_workspace_bytes(t.cfg, w.n_tokens, 5000) == 0
    t.close()


@pytest.mark.parametrize("geom,heads", [("deep", (0, 3)), ("light", (0,))])
def test_fit_at_bench_size(geom, heads):
    """The configuration bench.py --fit times: 32K tokens, 8 training queries per query head
    (64 per KV head), the workload's own reference queries; loss and gradient of the listed
    KV heads against the oracle (same tolerances)."""
    n, nq = 32_768, 8
    w = (wc.DEEP if geom == "deep" else wc.light(n)).with_(n_tokens=n, steps=1)
    K, V, refs = P.host_inputs(w)
    qs = np.stack([gen.step_queries(w, s, n, gen.host_fetch(K)) for s in range(nq)])
    refs32 = refs.astype(np.float32)
    t = P.make_tree(w)
    Kd, Vd = P.upload(K, w), P.upload(V, w)
    rt = torch.from_numpy(refs32).cuda()
    loss, grad = t.fit_step(Kd, Vd, n, rt, P.upload(qs, w), lr=0.0)
    loss, grad = loss.cpu().numpy(), grad.cpu().numpy()
    ro = oracle_refs(w, refs32)
    for kv in heads:
        qg = group_queries(w, qs, kv)
        lo, go = zo.fit_grad(K[kv], ro[kv], w.block, w.levels, n, qg)
        assert abs(loss[kv] - lo) <= 2e-4 * w.levels + 1e-5 * abs(lo), f"head {kv}: loss {loss[kv]:.6f} vs {lo:.6f}"
        allow = P.fit_flip_allowance(K[kv], ro[kv], w.block, w.levels, n, qg)
        err = np.abs(grad[kv] - go)
        tol = 2e-3 * np.max(np.abs(go)) + allow
        assert np.all(err <= tol), f"head {kv}: gradient error {np.max(err - tol):.3e} above tolerance"
    t.close()
