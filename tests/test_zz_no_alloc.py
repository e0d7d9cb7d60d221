"""The allocation-free dense decode (zha_decode_dense_static) through the C ABI against the
handle-based zha_decode_dense on the same inputs, and against the oracle: two calls in a row,
the second with a smaller input (fewer tokens, fewer heads, another head_dim)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import parity as P
from oracle import zha_oracle as zo
from workloads import configs as wc, gen

pytestmark = pytest.mark.gpu


def run_pair(w):
    from hierarchical_tree_indexed_03_amd import zha
    K, V, refs = P.host_inputs(w)
    Kd, Vd = P.upload(K, w), P.upload(V, w)
    t = P.make_tree(w)
    t.build(Kd, Vd, w.n_tokens, P.upload(refs, w))
    q = gen.step_queries(w, 3, w.n_tokens, gen.host_fetch(K))
    qd = P.upload(q, w)
    o_entry = t.decode_dense(qd)
    out = torch.full((w.num_q_heads, w.head_dim), float("nan"), dtype=torch.float32, device="cuda")
    zha.zha_decode_dense_static(t.cfg, Kd, Vd, w.n_tokens, qd, out)
    torch.cuda.synchronize()
    o_entry, out = o_entry.cpu().numpy(), out.cpu().numpy()
    assert np.all(np.isfinite(out))
    # same kernels; only the number of splits (hence the order of the final sums) may differ
    assert P.out_err(out, o_entry) <= 1e-4, f"static vs handle: {P.out_err(out, o_entry):.3e}"
    ref = zo.dense_decode(K, V, q, w.n_tokens)
    assert P.out_err(out, ref) <= P.OUT_RTOL, f"static vs oracle: {P.out_err(out, ref):.3e}"
    t.close()


def test_static_dense_two_calls():
    # first call: 32 query heads over 4 KV heads, d 128, 300K tokens (up to 252 splits per KV head)
    run_pair(wc.DEEP.with_(n_tokens=300_001, steps=0))
    # second call, smaller: 8 query heads over 2 KV heads, d 64, 5,003 tokens
    run_pair(wc.DEEP.with_(n_tokens=5_003, steps=0, num_kv_heads=2, num_q_heads=8, head_dim=64))
