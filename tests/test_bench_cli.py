"""bench.py on the host: it measures one GPU only and says so when asked for more."""
from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_every_decode_kernel_has_a_byte_model():
    """The bench's roofline reports whichever decode kernel is the longest; each of them needs
    algorithmic bytes, or the field would be null."""
    import numpy as np
    sys.path.insert(0, ROOT)
    import bench
    from workloads import configs as wc
    w = wc.DEEP
    n = w.n_tokens + 1
    rows = np.zeros((w.levels + 1, w.num_kv_heads), dtype=np.int64)
    for i in range(w.levels):
        rows[i] = w.nodes(w.levels - i, n)
    rows[w.levels] = 16_000
    for key_form in (True, False):
        for key in ("route_score.keys", "route_select.keys", "attend", "append", "route_prep", "route_score.top",
                    "route_score.l1", "dense_attend"):
            b = bench.kernel_bytes(key, w, rows, n, key_form)
            assert b is not None and b > 0, key
    # the keys route's scoring reads the keys and token weights once: about 0.39 GB at 256K
    assert 0.3e9 < bench.kernel_bytes("route_score.keys", w, rows, n, True) < 0.5e9
