"""Writes tiny_expected.json: the oracle's routed sets and outputs on the tiny workload
(1 KV head, head_dim 64, fp32, 4,096 keys, block 4, 3 levels, 4 reference queries,
p = 0.95, 8 planted queries).  Calls only the oracle and the seeded input generator.

    python tests/golden/make_golden.py
"""
from __future__ import annotations

import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from oracle import zha_oracle as zo  # noqa: E402
from workloads import configs as wc, gen  # noqa: E402

PATH = os.path.join(HERE, "tiny_expected.json")


def compute() -> dict:
    w = wc.TINY
    K, V = gen.kv_cache(w)
    refs = gen.ref_queries(w)
    tree = zo.build_tree(K[0], refs[0], w.block, w.levels, w.n_tokens)
    out = []
    for step in range(w.steps):
        q = gen.step_queries(w, step, w.n_tokens, gen.host_fetch(K))
        o, routes = zo.decode([tree], V, q, w.top_p, w.keep_sink, return_routes=True)
        r = routes[0]
        out.append(dict(step=step,
                        levels=[dict(level=int(lv["level"]), kept=[int(x) for x in lv["kept"]])
                                for lv in r["levels"]],
                        tokens=[int(x) for x in r["tokens"]],
                        out=[float(x) for x in o[0]]))
    return dict(workload=w.name, queries=out)


def load() -> dict:
    with open(PATH) as f:
        return json.load(f)


if __name__ == "__main__":
    with open(PATH, "w") as f:
        json.dump(compute(), f, indent=1)
    print("wrote", PATH)
