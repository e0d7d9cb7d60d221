"""Writes the routing trace of one decode step of the 16M-token ultra workload for the query
heads of KV head 0, for the CPU test that rebuilds that head's tree in the oracle
(tests/test_ultra_oracle_sets.py).

Runs on the GPU through the C ABI, in the launch configuration bench.py times: the tree is
built over the 16,777,216 seeded tokens, one token is appended, and the step's planted
queries are decoded.  Saved per level and query head of the group: the kept node ids, and
the GPU's scores of the frontier nodes within 2e-3 of the head's boundary score (the only
nodes a near-tie swap can involve); plus the queries and the outputs.

    python tests/data/make_ultra_trace.py <out.npz>
"""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

import parity as P  # noqa: E402
from workloads import configs as wc, gen  # noqa: E402

WINDOW = 2e-3


def main(path):
    w = wc.ULTRA.with_(steps=1)
    dt = P.torch_dtype(w)
    Kd = torch.empty(w.num_kv_heads, w.capacity, w.head_dim, dtype=dt, device="cuda")
    Vd = torch.empty_like(Kd)
    for s, h, lo, hi, rows in gen.iter_kv_chunks(w):
        (Kd if s == gen.STREAM_K else Vd)[h, lo:hi] = torch.from_numpy(rows).to(dt).cuda()
    print("[trace] caches uploaded", flush=True)
    refs = gen.ref_queries(w)
    t = P.make_tree(w)
    t.build(Kd, Vd, w.n_tokens, P.upload(refs, w))
    t.append(Kd[:, w.n_tokens].contiguous(), Vd[:, w.n_tokens].contiguous())
    n = w.n_tokens + 1
    fetch = lambda kv, idx: Kd[kv, torch.as_tensor(np.asarray(idx), device="cuda")].float().cpu().numpy()
    q = gen.step_queries(w, 0, n, fetch)
    o = t.decode(P.upload(q, w)).cpu().numpy()
    torch.cuda.synchronize()
    print("[trace] decoded", flush=True)
    rec = {"n_tokens": np.int64(n), "q": q[:w.group].astype(np.float32), "o": o[:w.group].astype(np.float32),
           "window": np.float64(WINDOW)}
    for lv in range(w.levels, -1, -1):
        tr = t.trace(lv)[0]                      # KV head 0
        for gi in range(w.group):
            if lv == 0:
                rec[f"blocks_g{gi}"] = P.gpu_frontier(tr, gi).astype(np.int32)
                continue
            fr = P.gpu_frontier(tr, gi)
            kept = P.gpu_kept(tr, gi)
            s = P.gpu_scores_on(tr, gi, fr)
            bnd = np.min(P.gpu_scores_on(tr, gi, kept))
            near = np.abs(s - bnd) <= WINDOW
            rec[f"kept_l{lv}_g{gi}"] = kept.astype(np.int32)
            rec[f"near_l{lv}_g{gi}"] = fr[near].astype(np.int32)
            rec[f"near_scores_l{lv}_g{gi}"] = s[near].astype(np.float32)
    np.savez_compressed(path, **rec)
    print(f"[trace] wrote {path} ({os.path.getsize(path)} bytes)", flush=True)
    t.close()


if __name__ == "__main__":
    main(sys.argv[1])
