"""The device invariant checks (libzha_debug.so: the same kernels with the checks compiled
in) stay silent over real decodes: build, appends, routed and dense decodes and a multi-token
append on the deep, ultra and light geometries at oracle-checked sizes.  Runs in a child
process that loads the debug library."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = r'''
import sys
sys.path.insert(0, ROOT); sys.path.insert(0, ROOT + "/tests")
import torch
import parity as P
from hierarchical_tree_indexed_03_amd import zha
from workloads import configs as wc, gen
assert zha.zha_debug_checks_compiled() == 1
for w in (wc.DEEP.with_(n_tokens=16_384 + 37, steps=3), wc.ULTRA.with_(n_tokens=70_001, steps=3),
          wc.light(288_003, steps=3).with_(num_kv_heads=1, num_q_heads=8)):
    K, V, refs = P.host_inputs(w)
    t = P.make_tree(w, capacity=w.capacity + 64)
    Kd, Vd = P.upload(K, w), P.upload(V, w)
    Kc = torch.zeros(w.num_kv_heads, w.capacity + 64, w.head_dim, dtype=Kd.dtype, device="cuda")
    Vc = torch.zeros_like(Kc)
    Kc[:, :w.capacity] = Kd
    Vc[:, :w.capacity] = Vd
    t.build(Kc, Vc, w.n_tokens, P.upload(refs, w))
    n = w.n_tokens
    for s in range(w.steps):
        t.append(Kc[:, n].contiguous(), Vc[:, n].contiguous())
        n += 1
        q = P.upload(gen.step_queries(w, s, n, gen.host_fetch(K)), w)
        t.decode(q)
        t.decode_dense(q)
    extra = torch.randn(w.num_kv_heads, 64, w.head_dim, device="cuda").to(Kd.dtype)
    t.append_n(extra, extra)
    t.decode(q)
    torch.cuda.synchronize()
    flags = zha.zha_debug_check(t.handle)
    print(w.name, "check flags", flags, flush=True)
    assert flags == 0, f"{w.name}: device checks failed: {flags:#x}"
    t.close()
print("DEBUG_CHECKS_OK", flush=True)
'''


def test_device_checks_silent():
    lib = os.path.join(ROOT, "hierarchical_tree_indexed_03_amd", "libzha_debug.so")
    assert os.path.exists(lib), "libzha_debug.so is not built (run __graft_entry__.build())"
    env = dict(os.environ, ZHA_LIB_PATH=lib)
    r = subprocess.run([sys.executable, "-c", f"ROOT = {ROOT!r}\n" + SCRIPT], capture_output=True, text=True,
                       env=env, timeout=280)
    print(r.stdout[-2000:])
    assert r.returncode == 0 and "DEBUG_CHECKS_OK" in r.stdout, (r.stdout + r.stderr)[-3000:]
