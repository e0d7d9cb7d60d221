"""Benchmark of the ZHA decode hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload deep]

A step is one pass of the whole decode path for one new token: zha_tree_append (one
key/value per KV head, refreshing the rightmost node of every level) then zha_decode (the
top-down top-p routing of all 32 query heads and the split-K attention over the routed
blocks plus the sink).  Inputs (caches, reference queries, the per-step queries and new
keys/values) are resident in HBM before the timed region.  The tree build over the
initial cache is timed separately (build tokens/s), as is the dense flash-decode over the
same cache (the baseline the method is compared with).

Prints one JSON line (the measurement record) on stdout.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from workloads import configs as wc, gen  # noqa: E402

METRIC = "ZHA decode queries/s per layer at 256K and 16M ctx; % HBM roofline; build tok/s"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0   # dense bf16 MFMA


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="deep", help="deep | wide | ultra | light_<N> | tiny")
    ap.add_argument("--planes", default="f32", choices=("f32", "bf16", "fp4"),
                    help="storage of the s vectors the router reads (bf16 / fp4: a quantised copy)")
    ap.add_argument("--p-levels", default=None,
                    help="per-level top-p schedule: p of levels 1..L comma-separated, or 'compound' "
                         "for p^(1/L) at every level (the product over the levels is p)")
    ap.add_argument("--no-quant-planes", "--no-bf16-planes", dest="no_quant_planes", action="store_true",
                    help="skip the secondary measurements with quantised (bf16, FP4) router planes")
    ap.add_argument("--append-chunk", type=int, default=4096,
                    help="also time zha_tree_append_n of this many tokens onto a tree of N-m (0: skip)")
    ap.add_argument("--build-reps", type=int, default=3)
    ap.add_argument("--dense-reps", type=int, default=20)
    ap.add_argument("--route", default="auto", choices=("auto", "frontier", "keys"),
                    help="decode scoring: the config's default, per-level union frontiers, or every level from the keys")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of timed oracle decode")
    ap.add_argument("--cold-steps", type=int, default=32,
                    help="extra steps timed one by one after a 1 GiB scratch write that evicts L2 and MALL")
    ap.add_argument("--crossover", action="store_true",
                    help="light-router sweep over N: ZHA vs dense decode, crossover context (own JSON line)")
    ap.add_argument("--prefill", action="store_true",
                    help="time the batched causal prefill alone (its own JSON line)")
    ap.add_argument("--prefill-tokens", type=int, default=64, help="tokens prefilled in --prefill")
    ap.add_argument("--prefill-batch", default="8,16,32,64", help="sub-batch sizes of --prefill")
    ap.add_argument("--fit", action="store_true",
                    help="reference-query fitting (zha_fit_step) at a 32K-token context on the deep and light "
                         "geometries: step time per stage, loss, routing before and after (own JSON line)")
    ap.add_argument("--fit-lr", type=float, default=1.0, help="SGD step of --fit")
    ap.add_argument("--fit-nq", type=int, default=8, help="training queries per query head and step in --fit")
    ap.add_argument("--cpu-sweep", action="store_true",
                    help="time the CPU oracle on the light sweep and the 16M workload (no GPU work)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration for traffic)")
    return ap.parse_args()


def node_bytes(w, level, key_form):
    """Algorithmic bytes read to score one union-frontier node at `level`: its R planes
    (R*(d+1) floats; with bf16 router planes R*d bf16 plus R float offsets; with MX FP4
    ones R*d/2 code bytes, R*d/32 scale bytes and R float offsets), or at level 1
    in key form its b keys (bf16) plus R*b token weights and R offsets; plus the 8-byte list
    entry and one float score per query head written."""
    R, d, g, b = w.num_ref, w.head_dim, w.group, w.block
    if level == 1 and key_form:
        core = b * d * 2 + R * b * 4 + R * 4
    elif w.planes == "bf16":
        core = R * d * 2 + R * 4
    elif w.planes == "fp4":
        core = R * (d // 2 + d // 32) + R * 4
    else:
        core = R * (d + 1) * 4
    return core + 8 + g * 4


TD_MAX = 33792   # the library's largest level selected top-down (scored whole)


def top_levels(w, n_tokens, key_form):
    """Levels scored whole and selected top-down: from the top down to the lowest level
    with at most TD_MAX nodes (level 1 excluded when it is scored in key form)."""
    lo = w.levels + 1
    while lo > 1 and w.nodes(lo - 1, n_tokens) <= TD_MAX:
        lo -= 1
    if key_form and lo == 1:
        lo = 2
    return list(range(lo, w.levels + 1))


AK_LC = 4   # the level whose nodes one all-keys score workgroup covers


def allkeys_score_bytes(w, n_tokens):
    """Algorithmic HBM bytes of one launch of the all-keys score kernel (every level from the
    keys): per KV head the N keys (bf16) and their level-1 token weights (R floats a token),
    each level-1..4 node's c and LSE (2R floats), one float score per query head written per
    node of levels 1..4, and the level-4 dot products (R floats per query head) written."""
    R, d, g = w.num_ref, w.head_dim, w.group
    per = n_tokens * (2 * d + 4 * R)
    for lv in range(1, AK_LC + 1):
        per += w.nodes(lv, n_tokens) * (8 * R + 4 * g)
    per += w.nodes(AK_LC, n_tokens) * g * R * 4
    return float(per * w.num_kv_heads)


def allkeys_upper_bytes(w, n_tokens):
    """Bytes the top-down selection reads to derive the levels above level 4: the level-4 dot
    products once per query head and each upper node's c and LSE once per query head."""
    R, g = w.num_ref, w.group
    per = w.nodes(AK_LC, n_tokens) * g * R * 4 * 2
    for lv in range(AK_LC + 1, w.levels + 1):
        per += w.nodes(lv, n_tokens) * 8 * R * g
    return float(per * w.num_kv_heads)


def allkeys_select_bytes(w, stats_rows, n_tokens):
    """Algorithmic HBM bytes of one launch of the top-down selection of the all-keys path:
    per query head the score rows of levels 1..4 (one float per node), the level-4 dot
    products and upper-level (c, LSE) it derives the levels above from, the upper levels'
    scores and every level's frontier and kept bitmaps written; per KV head the gather list
    of its kept blocks written (node id and head mask, 8 bytes a block)."""
    L, Hq = w.levels, w.num_q_heads
    per_head = sum(w.nodes(lv, n_tokens) * 4 for lv in range(1, AK_LC + 1))
    per_head += sum(w.nodes(lv, n_tokens) * 4 for lv in range(AK_LC + 1, L + 1))
    per_head += sum(2 * ((w.nodes(lv, n_tokens) + 31) // 32) * 4 for lv in range(1, L + 1))
    return float(per_head * Hq + allkeys_upper_bytes(w, n_tokens) + stats_rows[L].sum() * 8)


def append_bytes(w, key_form):
    """Algorithmic HBM bytes of one single-token append: the new K and V rows written, and at
    every level the rightmost node recomputed from its children (level 1: up to b keys, and
    the token weights in key form; above: up to b child planes) and written."""
    R, d, b, L = w.num_ref, w.head_dim, w.block, w.levels
    kb = 2 if w.dtype == "bf16" else 4
    plane = R * (d + 2) * 4                      # s, c and LSE of one node
    per = 2 * d * kb                             # the new K and V rows
    per += b * d * kb + plane + (R * b * 4 if key_form else 0)
    per += (L - 1) * (b * plane + plane)
    return float(per * w.num_kv_heads)


def kernel_bytes(key, w, stats_rows, n_tokens, key_form):
    """Algorithmic HBM bytes of one launch of `key` given the routing stats of that step.

    route_score.keys: allkeys_score_bytes; route_select.keys: allkeys_select_bytes;
    append: append_bytes; route_prep: q in, sigma*q out and the per-level state zeroed;
    route_score.l<l>: node_bytes per union-frontier node;
    route_score.top:  node_bytes per node of every top-down level (all of them are scored);
    attend:           per gathered token 2*d*2 bytes (K and V rows, bf16); partial results
                      excluded;
    dense_attend:     N * Hkv * 2 * d * 2 bytes.
    """
    d, L = w.head_dim, w.levels
    if key == "route_score.keys":
        return allkeys_score_bytes(w, n_tokens)
    if key == "route_select.keys":
        return allkeys_select_bytes(w, stats_rows, n_tokens)
    if key == "append":
        return append_bytes(w, key_form)
    if key == "route_prep":
        # q read (bf16), sigma*q written (fp32), per-level state zeroed
        return float(w.num_q_heads * w.head_dim * (2 + 4) + (w.levels + 1) * w.num_q_heads * 64)
    if key.startswith("route_score.l"):
        lv = int(key.split(".l")[1])
        u = stats_rows[L - lv].sum()
        return float(u) * node_bytes(w, lv, key_form)
    if key == "route_score.top":
        # every node of the top-down levels (their union-list counts are the level sizes)
        return float(sum(stats_rows[L - lv].sum() * node_bytes(w, lv, key_form) for lv in top_levels(w, n_tokens, key_form)))
    if key == "attend":
        blocks = stats_rows[L].sum()
        return float(blocks) * w.block * 2 * d * 2
    if key == "dense_attend":
        return float(n_tokens) * w.num_kv_heads * 2 * d * 2
    return None


def src_sha():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "hierarchical_tree_indexed_03_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".hpp")):
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_for(kernel, workload):
    """Measured HBM bytes per launch (FETCH_SIZE + WRITE_SIZE counters scaled by a plain copy)
    from the committed counter summary, if it was taken on the kernel's current sources."""
    from hierarchical_tree_indexed_03_amd.prof_summary import kernel_sha
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f).get("kernels", {}).get(kernel)
    if not t or t.get("src_sha") != kernel_sha(kernel):
        return None
    return t.get("bytes")


def cpu_baseline(w, K, V, refs, queries, n0, budget):
    """The oracle as written, timed on the host on a bounded sample: KV head 0's tree
    (built first, untimed, with every host thread), then decode steps of that head's query
    group on one thread (append + route + attend per step) until `budget` seconds."""
    from threadpoolctl import threadpool_limits
    from oracle import zha_oracle as zo
    tb0 = time.perf_counter()
    tree = zo.build_tree(K[0].copy(), refs[0], w.block, w.levels, n0)
    tb = time.perf_counter() - tb0
    steps = 0
    with threadpool_limits(1):
        t0 = time.perf_counter()
        while steps < len(queries) and time.perf_counter() - t0 < budget:
            if w.appends:
                zo.append_token(tree, K[0, tree.n_tokens])
            q = queries[steps]
            for h in range(w.group):
                r = zo.route(tree, q[h], w.top_p, w.keep_sink)
                zo.attend(tree.keys[:tree.n_tokens], V[0][:tree.n_tokens], q[h], r["tokens"])
            steps += 1
        el = time.perf_counter() - t0
    per_step_all_heads = el / max(steps, 1) * w.num_kv_heads
    return dict(value=1.0 / per_step_all_heads, unit="queries/s", cores=1, kind="oracle",
                sample=(f"KV head 0 of {w.num_kv_heads} (its {w.group} query heads), {steps} decode steps "
                        f"(append+route+attend) in {el:.1f}s on 1 thread, scaled x{w.num_kv_heads} to all "
                        f"heads; tree over {n0} tokens built first (untimed, {tb:.1f}s, all threads)"),
                host_cpus=os.cpu_count(), cpu_model=_cpu_model())


def _oracle_worker(args):
    """One KV head's query group on one host thread (a separate process): the oracle tree over
    the seeded cache, then append + route + attend steps of the group's planted queries until
    `budget` seconds.  Inputs are regenerated from the seeds in the process."""
    wname, n0, planes_f32, kv, budget, n_steps = args
    from threadpoolctl import threadpool_limits
    from oracle import zha_oracle as zo
    w = wc.NAMED[wname].with_(steps=n_steps)
    with threadpool_limits(1):
        K = gen.token_rows(w, gen.STREAM_K, kv, 0, n0 + n_steps)
        V = gen.token_rows(w, gen.STREAM_V, kv, 0, n0 + n_steps)
        refs = gen.ref_queries(w)[kv]
        tb0 = time.perf_counter()
        tree = zo.build_tree(K, refs, w.block, w.levels, n0)
        tb = time.perf_counter() - tb0
        fetch = lambda _kv, idx: K[idx]
        steps = 0
        t0 = time.perf_counter()
        while steps < n_steps and time.perf_counter() - t0 < budget:
            if w.appends:
                zo.append_token(tree, K[tree.n_tokens])
            for gi in range(w.group):
                q, _ = gen.planted_query(w, steps, kv * w.group + gi, tree.n_tokens, fetch)
                r = zo.route(tree, q, w.top_p, w.keep_sink)
                zo.attend(tree.keys[:tree.n_tokens], V[:tree.n_tokens], q, r["tokens"])
            steps += 1
        el = time.perf_counter() - t0
    return kv, steps, el, tb


def cpu_baseline_all_cores(w, n0, budget, n_steps):
    """The oracle on all host cores: one process per KV head (its query group), all at once,
    each on one thread; a step of the whole layer takes as long as the slowest process."""
    import multiprocessing as mp
    ctx = mp.get_context("spawn")
    jobs = [(w.name, n0, True, kv, budget, n_steps) for kv in range(w.num_kv_heads)]
    with ctx.Pool(len(jobs)) as pool:
        res = pool.map(_oracle_worker, jobs)
    per_step = max(el / max(st, 1) for _, st, el, _ in res)
    return dict(value=1.0 / per_step, unit="queries/s", cores=len(jobs), kind="oracle",
                sample=(f"{len(jobs)} processes at once, one per KV head (its {w.group} query heads) on one thread "
                        f"each; {min(st for _, st, _, _ in res)}-{max(st for _, st, _, _ in res)} decode steps "
                        f"(append+route+attend) in {budget:.0f}s each after building its tree "
                        f"({max(tb for *_, tb in res):.1f}s); a step = the slowest process's step time"),
                host_cpus=os.cpu_count(), cpu_model=_cpu_model())


def cpu_sweep(args):
    """The oracle on the light-router sweep (tree build plus 16 append+decode steps per N) and
    on the 16M-token workload (tree build plus 8 steps), for KV head 0's query group on one
    host thread, scaled to all KV heads.  The 16M tree is built level 1 chunk by chunk (the
    oracle's level-1 summary of a 2^20-token chunk is that of its blocks)."""
    from threadpoolctl import threadpool_limits
    from oracle import zha_oracle as zo
    rows = []
    cases = [(wc.light(n), 16) for n in wc.LIGHT_SIZES] + [(wc.ULTRA, 8)]
    for base, n_steps in cases:
        w = base.with_(steps=n_steps)
        n0 = w.n_tokens
        with threadpool_limits(1):
            refs = gen.ref_queries(w)[0].astype(np.float64)
            tb0 = time.perf_counter()
            s1, c1, K = [], [], []
            for lo in range(0, n0, gen.CHUNK):
                hi = min(n0, lo + gen.CHUNK)
                kr = gen.token_rows(w, gen.STREAM_K, 0, lo, hi)
                K.append(kr)
                s, c = zo.level1_planes(kr.astype(np.float64), refs, w.block)
                s1.append(s)
                c1.append(c)
            levels = [(np.concatenate(s1), np.concatenate(c1))]
            del s1, c1
            for _ in range(2, w.levels + 1):
                levels.append(zo.parent_planes(levels[-1][0], levels[-1][1], refs, w.block))
            tb = time.perf_counter() - tb0
            K.append(gen.token_rows(w, gen.STREAM_K, 0, n0, n0 + n_steps))
            K = np.concatenate(K)
            V = gen.token_rows(w, gen.STREAM_V, 0, 0, n0 + n_steps)     # untimed, like the keys
            tree = zo.Tree(keys=K, refs=refs, block=w.block, n_levels=w.levels, n_tokens=n0, levels=levels)
            fetch = lambda _kv, idx: K[idx]
            t0 = time.perf_counter()
            for st in range(n_steps):
                zo.append_token(tree, K[tree.n_tokens])
                for gi in range(w.group):
                    q, _ = gen.planted_query(w, st, gi, tree.n_tokens, fetch)
                    r = zo.route(tree, q, w.top_p, w.keep_sink)
                    tk = r["tokens"]
                    zo.attend(K[tk], V[tk], q, np.arange(len(tk)))
            el = time.perf_counter() - t0
        per_step = el / n_steps * w.num_kv_heads
        row = {"workload": w.name, "kv_tokens": n0, "oracle_build_s_one_kv_head": round(tb, 2),
               "oracle_build_tokens_per_s_all_heads": round(n0 / (tb * w.num_kv_heads), 1),
               "steps": n_steps, "oracle_step_s_all_heads": round(per_step, 3),
               "oracle_queries_per_s": round(1.0 / per_step, 4)}
        log(f"[cpu-sweep] {row}")
        rows.append(row)
        del tree, levels, K, V
    rec = {"metric": "oracle (CPU) build tokens/s and decode queries/s, light sweep and 16M",
           "unit": "queries/s", "cores": 1, "kind": "oracle", "host_cpus": os.cpu_count(), "cpu_model": _cpu_model(),
           "sample": ("KV head 0's query group on one host thread, scaled to all KV heads: the tree build "
                      "(the 16M one level 1 chunk by chunk), then append + route + attend steps; cache rows "
                      "generated from the seeds beforehand, untimed"),
           "per_workload": rows}
    print(json.dumps(rec), flush=True)


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def crossover(args):
    """ZHA step (append + decode) against dense flash-decode over the light-router sweep;
    warm (back to back) and cold (after a 1 GiB scratch write) per N.  Crossover = the
    smallest context where the ZHA step is faster, interpolated log-linearly in N."""
    import torch
    from hierarchical_tree_indexed_03_amd import zha
    dev = torch.device("cuda:0")
    steps = args.steps if args.steps is not None else 64
    rows = []
    scratch = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    for n0 in wc.LIGHT_SIZES:
        total = args.warmup + steps + args.cold_steps
        w = wc.light(n0, steps=total)
        Kd = torch.empty(w.num_kv_heads, w.capacity, w.head_dim, dtype=torch.bfloat16, device=dev)
        Vd = torch.empty_like(Kd)
        for stream, hh, lo, hi, r in gen.iter_kv_chunks(w):
            (Kd if stream == gen.STREAM_K else Vd)[hh, lo:hi] = torch.from_numpy(r).to(torch.bfloat16).to(dev)
        fetch = lambda kv, idx: Kd[kv, torch.as_tensor(idx, device=dev)].float().cpu().numpy()
        Qd = torch.from_numpy(np.stack([gen.step_queries(w, s_, n0 + s_ + 1, fetch) for s_ in range(total)])).to(torch.bfloat16).to(dev)
        Kn = Kd[:, n0:n0 + total].transpose(0, 1).contiguous()
        Vn = Vd[:, n0:n0 + total].transpose(0, 1).contiguous()
        Rd = torch.from_numpy(gen.ref_queries(w)).to(torch.bfloat16).to(dev)
        out = torch.empty(w.num_q_heads, w.head_dim, dtype=torch.float32, device=dev)
        zres = {}
        # the ZHA step with fp32 router planes, then with bf16 and FP4 copies (a tree each over
        # the same caches; their appends rewrite rows n0.. with the values they hold)
        for fmt in ("f32", "bf16", "fp4"):
            cfg = zha.make_config(w.head_dim, w.num_kv_heads, w.num_q_heads, w.block, w.levels, w.num_ref,
                                  w.capacity, w.dtype, w.top_p, w.keep_sink, fmt)
            tz = zha.Tree(cfg)
            tz.build(Kd, Vd, n0, Rd)

            def step(s_):
                tz.append(Kn[s_], Vn[s_])
                tz.decode(Qd[s_], out)

            for s_ in range(args.warmup):
                step(s_)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for s_ in range(args.warmup, args.warmup + steps):
                step(s_)
            e1.record()
            torch.cuda.synchronize()
            zw = e0.elapsed_time(e1) / steps
            zc = []
            for s_ in range(args.warmup + steps, total):
                scratch.fill_(float(s_))
                c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                c0.record()
                step(s_)
                c1.record()
                torch.cuda.synchronize()
                zc.append(c0.elapsed_time(c1))
            zres[fmt] = (zw, float(np.median(zc)) if zc else None)
            if fmt == "f32":
                tree = tz
            else:
                tz.close()
        zha_warm, zha_cold = zres["f32"]
        q_last = Qd[total - 1]
        for _ in range(3):
            tree.decode_dense(q_last, out)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.dense_reps):
            tree.decode_dense(q_last, out)
        e1.record()
        torch.cuda.synchronize()
        dense_warm = e0.elapsed_time(e1) / args.dense_reps
        dc = []
        for i in range(min(args.cold_steps, 16)):
            scratch.fill_(float(i))
            c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            c0.record()
            tree.decode_dense(q_last, out)
            c1.record()
            torch.cuda.synchronize()
            dc.append(c0.elapsed_time(c1))
        row = {"n_tokens": n0, "levels": w.levels, "zha_ms_warm": round(zha_warm, 4),
               "dense_ms_warm": round(dense_warm, 4),
               "zha_ms_cold_median": round(zha_cold, 4) if zha_cold else None,
               "dense_ms_cold_median": round(float(np.median(dc)), 4) if dc else None}
        for fmt in ("bf16", "fp4"):
            row[f"zha_ms_warm_{fmt}"] = round(zres[fmt][0], 4)
            row[f"zha_ms_cold_median_{fmt}"] = round(zres[fmt][1], 4) if zres[fmt][1] else None
        rows.append(row)
        log(f"[crossover] N={n0}: ZHA {row['zha_ms_warm']:.3f} ms warm / {row['zha_ms_cold_median']} cold "
            f"(bf16 planes {row['zha_ms_warm_bf16']:.3f}, FP4 {row['zha_ms_warm_fp4']:.3f} warm), "
            f"dense {row['dense_ms_warm']:.3f} ms warm / {row['dense_ms_cold_median']} cold")
        tree.close()
        del Kd, Vd, Kn, Vn, Qd
        torch.cuda.empty_cache()

    def cross(key_z, key_d):
        ns = np.array([r["n_tokens"] for r in rows], dtype=np.float64)
        rz = np.array([r[key_z] / r[key_d] if r[key_z] and r[key_d] else np.nan for r in rows])
        for i, r in enumerate(rz):
            if r < 1.0:
                if i == 0:
                    return {"tokens": None, "note": f"ZHA already faster at the smallest N ({int(ns[0])})"}
                lr0, lr1 = np.log(rz[i - 1]), np.log(r)
                t = (0.0 - lr0) / (lr1 - lr0)
                return {"tokens": round(float(np.exp(np.log(ns[i - 1]) + t * (np.log(ns[i]) - np.log(ns[i - 1]))))),
                        "between": [int(ns[i - 1]), int(ns[i])]}
        return {"tokens": None, "note": f"ZHA slower than dense at every N up to {int(ns[-1])}"}

    warm = cross("zha_ms_warm", "dense_ms_warm")
    cold = cross("zha_ms_cold_median", "dense_ms_cold_median")
    quant = {fmt: {"warm": cross(f"zha_ms_warm_{fmt}", "dense_ms_warm"),
                   "cold": cross(f"zha_ms_cold_median_{fmt}", "dense_ms_cold_median")} for fmt in ("bf16", "fp4")}
    rec = {"metric": "crossover context, ZHA decode step vs dense flash-decode (light router: R=1, b=8, p=0.75)",
           "value": warm.get("tokens"), "unit": "tokens", "n_gpus": 1, "steps": steps, "warmup": args.warmup,
           "higher_is_better": False, "data": "synthetic", "dtype": "bf16+f32",
           "config": {"workload": "light_sweep", "sizes": list(wc.LIGHT_SIZES), "kv_heads": 4, "q_heads": 32,
                      "head_dim": 128, "step": "append + decode"},
           "crossover_warm": warm, "crossover_cold": cold, "crossover_quantised_planes": quant, "per_n": rows,
           "modeled_reference": MODELED_REFERENCE}
    print(json.dumps(rec), flush=True)


# The pages' own speed figures: an H100 BF16 roofline model with trained reference queries,
# modeled rather than measured (blog "Zyphra Hierarchical Attention", section "How fast can
# ZHA get"; news summary "Zyphra releases the ZHA sparse attention method", section "How
# fast is ZHA?").
# Reported beside the measured line as context, never as the target of vs_baseline.
MODELED_REFERENCE = {"source": "the pages' H100 BF16 roofline model (modeled, not measured)",
                     "crossover_vs_dense_tokens": 48000, "crossover_vs_msa_tokens": 480000,
                     "speedup_vs_dense_256k": [1.93, 2.28], "speedup_vs_dense_10m": [32, 35]}


FIT_STAGES = ("fit.cast", "build", "fit.logits", "fit.mass", "fit.score", "fit.loss", "fit.alpha", "fit.grad")


def fit_stage_flops(stage, w, n, nq):
    """Algorithmic multiply-add work (as flops) of the MFMA stages: fit.score is
    2 Q R d flops per node of every level on fp32 MFMA; fit.logits 2 Q d per token (bf16)."""
    H, d, R, g = w.num_kv_heads, w.head_dim, w.num_ref, w.group
    Q = nq * g
    nodes = sum(-(-n // w.block ** lv) for lv in range(1, w.levels + 1))
    return {"fit.score": 2.0 * Q * R * d * nodes * H}.get(stage)


def fit_stage_bytes(stage, w, n, nq):
    """Algorithmic HBM bytes of one fitting stage (all KV heads), Q = nq * g queries per head:
    fit.logits  K once (2 B/element) + the logits z written (Q x N floats);
    fit.mass    z read once + the node log masses written (Q floats per node of every level);
    fit.score   every plane once (R (d+1) floats per node) + a score and an arg-max byte per
                (query, node);
    fit.loss    scores and log masses read, d loss / d score written, then read again with the
                arg-max bytes for the per-node sums (Q x 17 bytes per node);
    fit.alpha   K and z read once, alpha (R floats per token) written;
    fit.grad    K and alpha read once."""
    H, d, R, g = w.num_kv_heads, w.head_dim, w.num_ref, w.group
    Q = nq * g
    nodes = sum(-(-n // w.block ** lv) for lv in range(1, w.levels + 1))
    kbytes = n * d * 2
    per_head = {
        "fit.logits": kbytes + Q * n * 4,
        "fit.mass": Q * n * 4 + Q * nodes * 4,
        "fit.score": nodes * R * (d + 1) * 4 + Q * nodes * 5,
        "fit.loss": Q * nodes * (12 + 9) + nodes * R * 12,
        "fit.alpha": kbytes + Q * n * 4 + n * R * 4,
        "fit.grad": kbytes + n * R * 4,
    }.get(stage)
    return None if per_head is None else float(per_head * H)


def fit_bench(args):
    """Reference-query fitting with zha_fit_step at a 32K-token context (the pages fit at 32K)
    on the deep geometry (b 4, L 6, R 16) and the light router (R 1, b 8).  Per geometry:
    `steps` SGD steps on planted training queries (nq per query head, new ones every step),
    timed as a whole and stage by stage; the loss before and after; and routing on held-out
    planted queries with the initial and the fitted reference queries (kept blocks of the
    union, and the relative distance of the routed output to dense decode)."""
    import torch
    from hierarchical_tree_indexed_03_amd import zha
    dev = torch.device("cuda:0")
    n = 32_768
    steps = args.steps if args.steps is not None else 40
    nq = args.fit_nq
    n_eval = 16
    res = []
    for base in (wc.DEEP, wc.light(n)):
        w = base.with_(n_tokens=n, steps=1)
        dt = torch.bfloat16
        K, V = gen.kv_cache(w)
        Kd, Vd = (torch.from_numpy(x).to(dt).to(dev) for x in (K, V))
        fetch = gen.host_fetch(K)
        train_h = np.stack([gen.step_queries(w, s_, n, fetch) for s_ in range(steps * nq)])
        train = torch.from_numpy(train_h).to(dt).to(dev)
        held = torch.from_numpy(np.stack([gen.step_queries(w, 100_000 + s_, n, fetch) for s_ in range(n_eval)])).to(dt).to(dev)
        cpu = None
        if not args.no_cpu and not res:
            # the oracle's fit_grad on KV head 0 with its group's first batch of queries (one
            # query per head), on one thread, scaled to a whole step (nq per head, all heads)
            from threadpoolctl import threadpool_limits
            from oracle import zha_oracle as zo
            r0 = gen.ref_queries(w)[0].astype(np.float64)
            calls = 0
            with threadpool_limits(1):
                c0 = time.perf_counter()
                while calls < len(train_h) and time.perf_counter() - c0 < min(args.cpu_budget, 10.0):
                    zo.fit_grad(K[0], r0, w.block, w.levels, n, train_h[calls, :w.group, :].astype(np.float64))
                    calls += 1
                el = time.perf_counter() - c0
            per_step = el / calls * nq * w.num_kv_heads
            cpu = {"value": round(per_step * 1e3, 1), "unit": "ms/step", "cores": 1, "kind": "oracle",
                   "sample": (f"oracle.fit_grad on KV head 0 of {w.num_kv_heads}, {calls} calls with {w.group} training "
                              f"queries each (one per query head) over {n} tokens: {el:.1f}s on 1 thread, scaled to a "
                              f"step of {nq} queries per query head on every KV head"),
                   "host_cpus": os.cpu_count(), "cpu_model": _cpu_model()}
        del K, V
        refs0 = torch.from_numpy(gen.ref_queries(w)).float().to(dev)
        cfg = zha.make_config(w.head_dim, w.num_kv_heads, w.num_q_heads, w.block, w.levels, w.num_ref, n,
                              w.dtype, w.top_p, w.keep_sink)
        t = zha.Tree(cfg)
        out = torch.empty(w.num_q_heads, w.head_dim, dtype=torch.float32, device=dev)
        dense = torch.empty_like(out)
        stats = torch.zeros(w.levels + 1, w.num_kv_heads, dtype=torch.int32, device=dev)

        def route_eval(refs):
            rb = refs.to(dt).contiguous()
            t.build(Kd, Vd, n, rb)
            kept, err = [], []
            for e_ in range(n_eval):
                t.decode(held[e_], out, stats)
                t.decode_dense(held[e_], dense)
                kept.append(int(stats[w.levels].sum().item()))
                err.append(float(((out - dense).norm(dim=1) / dense.norm(dim=1)).mean().item()))
            return dict(kept_blocks_union=float(np.mean(kept)), blocks=int(-(-n // w.block)) * w.num_kv_heads,
                        out_rel_err_vs_dense=float(np.mean(err)))

        before = route_eval(refs0)
        refs = refs0.clone()
        loss0, _ = t.fit_step(Kd, Vd, n, refs, train[:nq], lr=0.0, grad=False)
        loss0 = float(loss0.mean().item())
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for s_ in range(steps):
            t.fit_step(Kd, Vd, n, refs, train[s_ * nq:(s_ + 1) * nq], lr=args.fit_lr, grad=False)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        loss1, _ = t.fit_step(Kd, Vd, n, refs, train[:nq], lr=0.0, grad=False)
        loss1 = float(loss1.mean().item())
        # per-stage times (lr = 0: the fitted queries stay as they are)
        stage_ms = {}
        for key in FIT_STAGES:
            zha.zha_profile_start(t.handle, key)
            for s_ in range(4):
                t.fit_step(Kd, Vd, n, refs, train[s_ * nq:(s_ + 1) * nq], lr=0.0, grad=False)
            torch.cuda.synchronize()
            tot, cnt = zha.zha_profile_stop(t.handle)
            stage_ms[key] = tot / 4
        after = route_eval(refs)
        dom = max((k for k in stage_ms if k.startswith("fit.")), key=stage_ms.get)
        fl = fit_stage_flops(dom, w, n, nq)
        bts = fit_stage_bytes(dom, w, n, nq)
        roof = None
        if fl is not None:
            ach = fl / (stage_ms[dom] * 1e-3) / 1e12
            roof = {"bound": "mfma", "kernel": dom, "achieved": round(ach, 2), "peak": 157.3, "unit": "TFLOP/s",
                    "dtype": "f32", "frac": round(ach / 157.3, 4), "algorithmic_flops_per_step": fl,
                    "algorithmic_bytes_per_step": bts, "avg_stage_ms": round(stage_ms[dom], 4), "traffic": None}
        elif bts is not None:
            ach = bts / (stage_ms[dom] * 1e-3) / 1e9
            roof = {"bound": "hbm", "kernel": dom, "achieved": round(ach, 1), "peak": 8000.0, "unit": "GB/s",
                    "frac": round(ach / 8000.0, 4), "algorithmic_bytes_per_step": bts,
                    "avg_stage_ms": round(stage_ms[dom], 4), "traffic": None}
        Q = nq * w.group
        row = {"geometry": w.name.split("_")[0], "n_tokens": n, "block": w.block, "levels": w.levels,
               "num_ref": w.num_ref, "top_p": w.top_p, "train_queries_per_kv_head_per_step": Q, "steps": steps,
               "lr": args.fit_lr, "ms_per_step": round(ms, 4),
               "train_queries_per_s": round(Q * w.num_kv_heads / (ms * 1e-3), 1),
               "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()}, "roofline": roof,
               "loss_first_batch": {"before": round(loss0, 4), "after": round(loss1, 4)},
               "held_out_routing": {"initial_refs": before, "fitted_refs": after}, "cpu_baseline": cpu}
        log(f"[fit] {row['geometry']}: {ms:.3f} ms/step ({row['train_queries_per_s']:.0f} training queries/s), "
            f"loss {loss0:.3f} -> {loss1:.3f}; held-out kept blocks {before['kept_blocks_union']:.0f} -> "
            f"{after['kept_blocks_union']:.0f}, output error vs dense {before['out_rel_err_vs_dense']:.4f} -> "
            f"{after['out_rel_err_vs_dense']:.4f}; stages " + ", ".join(f"{k}={v:.3f}" for k, v in stage_ms.items()))
        res.append(row)
        t.close()
        del Kd, Vd, train, held
        torch.cuda.empty_cache()
    top = res[0]
    rec = {"metric": "reference-query fit step time (zha_fit_step, KL to dense node mass at every level)",
           "value": top["ms_per_step"], "unit": "ms/step", "n_gpus": 1, "steps": steps, "warmup": 0,
           "higher_is_better": False, "vs_baseline": None, "data": "synthetic (planted queries)",
           "dtype": "bf16+f32", "config": {"workload": "fit_32k", "geometries": [r["geometry"] for r in res]},
           "roofline": top["roofline"], "cpu_baseline": top["cpu_baseline"], "per_geometry": res}
    print(json.dumps(rec))


def prefill_legs(zha, tree, w, Kd, Vd, Qd, Rd, n0, mp, batches, dev):
    """Causal prefill of the mp tokens before n0 onto a tree built over n0 - mp: the
    per-token loop (zha_prefill: append + routed decode per token) once, then the batched
    prefill (zha_prefill_batched) at each sub-batch size: median of 3 timed runs, the time of
    each stage (HIP events around its launches in a separate run), and the scoring pass
    against its bounds.  Inputs resident in HBM; every run starts from a fresh build
    (untimed).  Returns (per_token, batched)."""
    import torch
    R, d, g, L = w.num_ref, w.head_dim, w.group, w.levels
    Kc, Vc = Kd[:, n0 - mp:n0].contiguous(), Vd[:, n0 - mp:n0].contiguous()
    Qc = Qd[:mp].contiguous()
    pout = torch.empty(mp, w.num_q_heads, d, dtype=torch.float32, device=dev)

    def timed(fn):
        tree.build(Kd, Vd, n0 - mp, Rd)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    timed(lambda: tree.prefill(Kc, Vc, Qc, pout))
    pm = timed(lambda: tree.prefill(Kc, Vc, Qc, pout))
    per_token = {"tokens": mp, "onto_tokens": n0 - mp, "ms": round(pm, 4), "ms_per_token": round(pm / mp, 4),
                 "tokens_per_s": round(mp / (pm * 1e-3), 1)}
    log(f"[bench] prefill of {mp} tokens (append + decode each): {pm:.3f} ms, {pm / mp:.4f} ms/token")
    pout2 = torch.empty_like(pout)
    batched = {}
    nodes_all = sum(-(-n0 // w.block ** l) for l in range(1, L + 1))
    for bt in batches:
        if bt > mp:
            continue
        timed(lambda: tree.prefill_batched(Kc, Vc, Qc, bt, out=pout2))
        bm = float(np.median([timed(lambda: tree.prefill_batched(Kc, Vc, Qc, bt, out=pout2)) for _ in range(3)]))
        stage = {}
        for key in ("prefill_prep", "prefill_score", "prefill_select", "prefill_attend", "build_tile"):
            tree.build(Kd, Vd, n0 - mp, Rd)
            torch.cuda.synchronize()
            zha.zha_profile_start(tree.handle, key)
            tree.prefill_batched(Kc, Vc, Qc, bt, out=pout2)
            torch.cuda.synchronize()
            ms_, _ = zha.zha_profile_stop(tree.handle)
            stage[key] = round(ms_, 4)
        # the scoring pass against its bounds: every node's planes read once per sub-batch,
        # 2 R d flops per (pair, node) counted in float32 (each computed as three bf16 MFMA
        # products, so the MFMA ceiling for it is a third of the bf16 peak)
        nsub = -(-mp // bt)
        sb = w.num_kv_heads * nodes_all * R * (d + 1) * 4
        sf = sum(2.0 * w.num_kv_heads * min(bt, mp - i * bt) * g * nodes_all * R * d for i in range(nsub))
        sms = stage["prefill_score"] / nsub
        score = {"ms_per_sub_batch": round(sms, 4), "alg_bytes": round(sb),
                 "achieved_GBps": round(sb / (sms * 1e-3) / 1e9, 1),
                 "frac_hbm": round(sb / (sms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                 "fp32_TFLOPs": round(sf / nsub / (sms * 1e-3) / 1e12, 2),
                 "frac_bf16_mfma_third": round(sf / nsub / (sms * 1e-3) / 1e12 / (BF16_PEAK_TFLOPS / 3), 4),
                 "note": "score + tail launches per sub-batch (the tail is ~2% of it)"}
        batched[str(bt)] = {"ms": round(bm, 4), "tokens_per_s": round(mp / (bm * 1e-3), 1),
                            "speedup_vs_per_token": round(pm / bm, 3), "stage_ms": stage, "score": score,
                            "max_abs_diff_vs_per_token": round(float((pout2 - pout).abs().max()), 6)}
        log(f"[bench] batched prefill of {mp} tokens, {bt} per sub-batch: {bm:.3f} ms "
            f"({mp / (bm * 1e-3):.0f} tok/s, {pm / bm:.2f}x the per-token loop); stages " +
            ", ".join(f"{k}={v:.3f}" for k, v in stage.items()))
    return per_token, batched


def prefill_bench(args):
    """`--prefill`: the batched causal prefill alone on one workload (deep by default): the
    last `--prefill-tokens` tokens of the cache prefilled onto a tree over the rest, per
    token and in sub-batches of each `--prefill-batch` size.  Prints its own JSON line."""
    import torch
    from hierarchical_tree_indexed_03_amd import zha
    w = wc.NAMED[args.workload].with_(steps=0, appends=False)
    n0, mp = w.n_tokens, args.prefill_tokens
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    Kd = torch.empty(w.num_kv_heads, w.capacity, w.head_dim, dtype=tdt, device=dev)
    Vd = torch.empty_like(Kd)
    for stream, hh, lo, hi, rows in gen.iter_kv_chunks(w):
        (Kd if stream == gen.STREAM_K else Vd)[hh, lo:hi] = torch.from_numpy(rows).to(tdt).to(dev)
    fetch = lambda kv, idx: Kd[kv, torch.as_tensor(idx, device=dev)].float().cpu().numpy()
    Qd = torch.from_numpy(np.stack([gen.step_queries(w, s_, n0 - mp + s_ + 1, fetch) for s_ in range(mp)])).to(tdt).to(dev)
    Rd = torch.from_numpy(gen.ref_queries(w)).to(tdt).to(dev)
    cfg = zha.make_config(w.head_dim, w.num_kv_heads, w.num_q_heads, w.block, w.levels, w.num_ref,
                          w.capacity, w.dtype, w.top_p, w.keep_sink, w.planes)
    tree = zha.Tree(cfg)
    batches = tuple(int(x) for x in args.prefill_batch.split(","))
    per_token, batched = prefill_legs(zha, tree, w, Kd, Vd, Qd, Rd, n0, mp, batches, dev)
    best = max(batched.values(), key=lambda r: r["tokens_per_s"])
    rec = {"metric": "ZHA batched causal prefill tokens/s per layer", "value": best["tokens_per_s"],
           "unit": "tokens/s", "n_gpus": 1, "higher_is_better": True, "dtype": "bf16+f32", "data": "synthetic",
           "config": {"workload": f"{w.name}_{n0}_prefill{mp}", "kv_tokens": n0, "prefill_tokens": mp,
                      "head_dim": w.head_dim, "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads,
                      "block": w.block, "levels": w.levels, "num_ref": w.num_ref, "top_p": w.top_p},
           "per_token_loop": per_token, "batched": batched, "src_sha": src_sha()}
    print(json.dumps(rec), flush=True)
    tree.close()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the path has no multi-GPU mode", file=sys.stderr)
        sys.exit(2)

    import torch
    from hierarchical_tree_indexed_03_amd import zha

    if args.cpu_sweep:
        return cpu_sweep(args)
    if args.crossover:
        return crossover(args)
    if args.fit:
        return fit_bench(args)
    if args.prefill:
        return prefill_bench(args)
    base = wc.NAMED[args.workload]
    steps = args.steps if args.steps is not None else (base.steps or 64)
    # extra steps after the cold ones: the dominant kernel timed with HIP events around each
    # launch (events inside the timed steps would add their own gaps to `value`)
    ksteps = min(steps, 64)
    total = args.warmup + steps + args.cold_steps + ksteps
    w = base.with_(steps=total, planes=args.planes)
    n0 = w.n_tokens
    prof_name = w.name if w.planes == "f32" else f"{w.name}_{w.planes}planes"   # counter summaries
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = torch.device("cuda:0")

    t = time.perf_counter()
    Kd = torch.empty(w.num_kv_heads, w.capacity, w.head_dim, dtype=tdt, device=dev)
    Vd = torch.empty_like(Kd)
    for stream, hh, lo, hi, rows in gen.iter_kv_chunks(w):
        (Kd if stream == gen.STREAM_K else Vd)[hh, lo:hi] = torch.from_numpy(rows).to(tdt).to(dev)
    torch.cuda.synchronize()
    refs = gen.ref_queries(w)

    def fetch(kv, idx):
        return Kd[kv, torch.as_tensor(idx, device=dev)].float().cpu().numpy()

    queries = np.stack([gen.step_queries(w, s, n0 + s + (1 if w.appends else 0), fetch) for s in range(total)])
    log(f"[bench] inputs generated in {time.perf_counter() - t:.1f}s: {w.name} N={n0} steps={steps} warmup={args.warmup}")

    Rd = torch.from_numpy(refs).to(tdt).to(dev)
    Qd = torch.from_numpy(queries).to(tdt).to(dev)                    # [steps, Hq, d]
    Kn = Kd[:, n0:n0 + total].transpose(0, 1).contiguous()            # [steps, Hkv, d]
    Vn = Vd[:, n0:n0 + total].transpose(0, 1).contiguous()
    out = torch.empty(w.num_q_heads, w.head_dim, dtype=torch.float32, device=dev)
    stats = torch.zeros(total, w.levels + 1, w.num_kv_heads, dtype=torch.int32, device=dev)

    cfg = zha.make_config(w.head_dim, w.num_kv_heads, w.num_q_heads, w.block, w.levels, w.num_ref,
                          w.capacity, w.dtype, w.top_p, w.keep_sink, w.planes)
    tree = zha.Tree(cfg)
    h = tree.handle
    key_form = zha.zha_level1_key_form(cfg) == 1
    tree.set_route_mode({"auto": 0, "frontier": 1, "keys": 2}[args.route])
    allkeys = tree.route_mode == 2
    p_levels = None
    if args.p_levels:
        p_levels = ([w.top_p ** (1.0 / w.levels)] * w.levels if args.p_levels == "compound"
                    else [float(x) for x in args.p_levels.split(",")])
        tree.set_top_p_levels(p_levels)

    # ---- tree build (timed separately; the last build is the one decoded against)
    torch.cuda.synchronize()
    build_ms = []
    for _ in range(max(1, args.build_reps)):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        tree.build(Kd, Vd, n0, Rd)
        e1.record()
        torch.cuda.synchronize()
        build_ms.append(e0.elapsed_time(e1))
    build_s = min(build_ms) / 1e3
    build_tok_s = n0 / build_s
    # read the keys once; write every plane (plus the bf16 router copies of s, and the
    # level-1 token weights in key form) once
    copies = [l for l in range(1, w.levels + 1) if w.planes != "f32" and not (l == 1 and key_form)]
    copy_b = {"f32": 0, "bf16": w.head_dim * 2, "fp4": w.head_dim // 2 + w.head_dim // 32}[w.planes]
    build_bytes = n0 * w.num_kv_heads * (w.head_dim * (2 if w.dtype == "bf16" else 4) +
                                        sum(w.num_ref * (w.head_dim + 1) * 4 / w.block ** l
                                            for l in range(1, w.levels + 1)) +
                                        sum(w.num_ref * copy_b / w.block ** l for l in copies) +
                                        (w.num_ref * 4 if key_form else 0))
    log(f"[bench] build {build_s * 1e3:.3f} ms -> {build_tok_s / 1e9:.3f} G tok/s")

    def step(s):
        if w.appends:
            tree.append(Kn[s], Vn[s])
        tree.decode(Qd[s], out, stats[s])

    # ---- warmup
    zha.zha_profile_start(h, "append")
    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    app_ms, app_n = zha.zha_profile_stop(h)
    # rank the launches of one extra (untimed, append-free) decode; one bracket per decode
    # keeps each launch's timing undisturbed by the other brackets
    keys = ["route_prep", "attend", "route_score.top", "route_select.top", "route_expand.top",
            "route_score.keys", "route_select.keys", "route_expand.keys"] + [
        f"route_{k}.l{l}" for l in range(1, w.levels + 1) for k in ("score", "select", "expand")]
    probe_ms = {}
    snap = tree.n_tokens
    for key in keys:
        zha.zha_profile_start(h, key)
        tree.decode(Qd[min(args.warmup, total - 1)], out, None)
        torch.cuda.synchronize()
        ms, n = zha.zha_profile_stop(h)
        probe_ms[key] = ms / max(n, 1)
    assert tree.n_tokens == snap
    if app_n:
        probe_ms["append"] = app_ms / app_n
    dominant = max(probe_ms, key=probe_ms.get)
    log("[bench] per-launch ms: " + ", ".join(f"{k}={v:.4f}" for k, v in sorted(probe_ms.items(), key=lambda x: -x[1])[:8]))

    # ---- timed region
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for s in range(args.warmup, args.warmup + steps):
        step(s)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1)
    ms_per_step = wall * 1e3 / steps
    qps = steps / wall
    st = stats.cpu().numpy()
    timed_stats = st[args.warmup:args.warmup + steps]
    # every decode kernel against the HBM roofline (per-launch times of the probe decode above,
    # algorithmic bytes at the first timed step's routing stats), for the dominant one's context
    kernel_roofline = {}
    for key, ms in sorted(probe_ms.items(), key=lambda x: -x[1]):
        if ms <= 0:
            continue
        kb = kernel_bytes(key, w, timed_stats[0], n0 + args.warmup + 1, key_form)
        if kb is None:
            continue
        kernel_roofline[key] = {"ms": round(ms, 4), "alg_bytes": round(kb),
                                "frac_hbm": round(kb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    log(f"[bench] timed {steps} steps: {ms_per_step:.3f} ms/step (events {gpu_ms / steps:.3f}), "
        f"{qps:.1f} queries/s")

    # ---- cold steps: before each (outside its timing) the caches are evicted.  Primary: a
    # 2 GiB streaming read of another buffer fills L2 and the Infinity Cache with clean
    # lines, as the other layers' caches would between two decode steps of this layer.
    # Also reported: a 1 GiB scratch write instead, which leaves 256 MB of dirty lines that
    # the step's first misses must write back.
    import ctypes
    plib = ctypes.CDLL(os.path.join(ROOT, "hierarchical_tree_indexed_03_amd", "libzha_probe.so"))
    plib.zha_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    plib.zha_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    cold = None
    cold_write = None
    n_cold_read = (args.cold_steps + 1) // 2
    if args.cold_steps > 0:
        sst = torch.cuda.current_stream().cuda_stream
        flush_b = 1 << 31
        flush_buf = torch.zeros(flush_b, dtype=torch.uint8, device=dev)
        flush_sink = torch.empty(4096, dtype=torch.int32, device=dev)
        cold_ms, cold_w_ms = [], []
        for i_, s_ in enumerate(range(args.warmup + steps, args.warmup + steps + args.cold_steps)):
            by_read = i_ < n_cold_read
            if by_read:
                plib.zha_probe_stream_read(flush_buf.data_ptr(), flush_b, flush_sink.data_ptr(), 1024, sst)
            else:
                flush_buf[:1 << 30].fill_(s_ & 0xff)
            c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            c0.record()
            step(s_)
            c1.record()
            torch.cuda.synchronize()
            (cold_ms if by_read else cold_w_ms).append(c0.elapsed_time(c1))
        del flush_buf
        cm = np.array(cold_ms)
        cold = {"flush": "2 GiB streaming read of another buffer before each step", "steps": len(cm),
                "median_ms": round(float(np.median(cm)), 4), "p90_ms": round(float(np.percentile(cm, 90)), 4),
                "queries_per_s_median": round(1e3 / float(np.median(cm)), 2)}
        if cold_w_ms:
            cw = np.array(cold_w_ms)
            cold_write = {"flush": "1 GiB scratch write before each step", "steps": len(cw),
                          "median_ms": round(float(np.median(cw)), 4), "p90_ms": round(float(np.percentile(cw, 90)), 4)}
        log(f"[bench] cold steps: median {cold['median_ms']:.3f} ms, p90 {cold['p90_ms']:.3f} ms"
            + (f"; after a scratch write instead: median {cold_write['median_ms']:.3f} ms" if cold_write else ""))

    # ---- the dominant kernel, timed live: HIP events around each of its launches (on the
    # stream it runs on) over ksteps more steps of the same workload
    k0 = args.warmup + steps + args.cold_steps
    zha.zha_profile_start(h, dominant)
    for s_ in range(k0, k0 + ksteps):
        step(s_)
    torch.cuda.synchronize()
    dom_ms, dom_n = zha.zha_profile_stop(h)
    kst = stats.cpu().numpy()[k0:k0 + ksteps]
    dom_bytes = [kernel_bytes(dominant, w, kst[i], n0 + k0 + i + 1, key_form) for i in range(ksteps)]
    dom_avg_ms = dom_ms / max(dom_n, 1)
    roofline = None
    if dom_bytes[0] is not None:
        alg = float(np.mean(dom_bytes))
        achieved = alg / (dom_avg_ms * 1e-3) / 1e9
        roofline = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                        frac=round(achieved / HBM_PEAK_GBS, 4), traffic=traffic_for(dominant, prof_name),
                        kernel=dominant, launches=dom_n, avg_launch_ms=round(dom_avg_ms, 4),
                        algorithmic_bytes_per_launch=round(alg))
    log(f"[bench] dominant {dominant}: {dom_avg_ms:.4f} ms/launch over {dom_n} launches")

    # ---- decode-step bytes (router planes + gathered KV), from the routing stats
    R, d, g, L = w.num_ref, w.head_dim, w.group, w.levels
    per_level = np.array([node_bytes(w, L - row, key_form) for row in range(L)], dtype=np.float64)
    router_b = (timed_stats[:, :L, :].sum(axis=2) * per_level[None, :]).sum(axis=1)
    if allkeys:
        router_b = np.array([allkeys_score_bytes(w, n0 + args.warmup + i + 1) + allkeys_upper_bytes(w, n0 + args.warmup + i + 1)
                             for i in range(steps)])
    gather_b = timed_stats[:, L, :].sum(axis=1) * w.block * 2 * d * 2
    step_bytes = float(np.mean(router_b + gather_b))
    # the whole step against the HBM roofline: cold first (each step after the read flush),
    # then warm (the timed steps back to back, the `value` line)
    roofline_step = None
    if cold:
        cst = stats.cpu().numpy()[args.warmup + steps:args.warmup + steps + n_cold_read]
        c_router = (cst[:, :L, :].sum(axis=2) * per_level[None, :]).sum(axis=1)
        if allkeys:
            c_router = np.array([allkeys_score_bytes(w, n0 + args.warmup + steps + i + 1) +
                                 allkeys_upper_bytes(w, n0 + args.warmup + steps + i + 1) for i in range(len(cst))])
        cold_bytes = float(np.mean(c_router + cst[:, L, :].sum(axis=1) * w.block * 2 * d * 2))
        ach_c = cold_bytes / (cold["median_ms"] * 1e-3) / 1e9
        ach_w = step_bytes / (ms_per_step * 1e-3) / 1e9
        roofline_step = {
            "bound": "hbm", "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "cold": {"achieved": round(ach_c, 1), "frac": round(ach_c / HBM_PEAK_GBS, 4), "ms": cold["median_ms"],
                     "alg_bytes": round(cold_bytes)},
            "warm": {"achieved": round(ach_w, 1), "frac": round(ach_w / HBM_PEAK_GBS, 4), "ms": round(ms_per_step, 4),
                     "alg_bytes": round(step_bytes)},
            "note": ("whole append+decode step: router bytes of the union frontiers plus the gathered K/V over the "
                     "step time; cold = median step after a cache-evicting read.  `value` is the warm rate because "
                     "the timed region is K consecutive steps between two synchronisations, which leaves no room "
                     "for a flush between steps")}
        log(f"[bench] step roofline: cold {ach_c:.0f} GB/s ({ach_c / HBM_PEAK_GBS:.3f}), warm {ach_w:.0f} GB/s "
            f"({ach_w / HBM_PEAK_GBS:.3f})")

    # ---- dense flash-decode over the same cache (baseline)
    q_last = Qd[args.warmup + steps - 1]
    for _ in range(3):
        tree.decode_dense(q_last, out)
    torch.cuda.synchronize()
    zha.zha_profile_start(h, "dense_attend")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.dense_reps):
        tree.decode_dense(q_last, out)
    e1.record()
    torch.cuda.synchronize()
    dense_ms_k, dense_n = zha.zha_profile_stop(h)
    dense_ms = e0.elapsed_time(e1) / args.dense_reps
    dense_bytes = tree.n_tokens * w.num_kv_heads * 2 * d * 2
    log(f"[bench] dense decode {dense_ms:.3f} ms ({dense_bytes / dense_ms / 1e6:.0f} GB/s)")

    # ---- the same warm steps with quantised router planes (bf16, MX FP4): a second tree
    # over the same caches (its appends rewrite rows n0.. with the values they already hold)
    quant = {}
    legs = ("bf16", "fp4") if w.planes == "f32" and not args.no_quant_planes else ()
    if allkeys and not args.no_quant_planes:
        legs = ("f32",) + legs     # the frontier path, which reads the planes, for comparison
    for fmt in legs:
        w2 = w.with_(planes=fmt)
        cfg2 = zha.make_config(w.head_dim, w.num_kv_heads, w.num_q_heads, w.block, w.levels, w.num_ref,
                               w.capacity, w.dtype, w.top_p, w.keep_sink, fmt)
        tree2 = zha.Tree(cfg2)
        if allkeys:
            tree2.set_route_mode(1)
        if p_levels:
            tree2.set_top_p_levels(p_levels)
        b_ms = []
        for _ in range(max(1, args.build_reps)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            tree2.build(Kd, Vd, n0, Rd)
            e1.record()
            torch.cuda.synchronize()
            b_ms.append(e0.elapsed_time(e1))
        stats2 = torch.zeros_like(stats)

        def step2(s_):
            if w.appends:
                tree2.append(Kn[s_], Vn[s_])
            tree2.decode(Qd[s_], out, stats2[s_])
        for s_ in range(args.warmup):
            step2(s_)
        probe2 = {}
        for key in ("route_score.top", "route_score.l1", "route_score.l2", "attend"):
            zha.zha_profile_start(tree2.handle, key)
            tree2.decode(Qd[min(args.warmup, total - 1)], out, None)
            torch.cuda.synchronize()
            ms_, n_ = zha.zha_profile_stop(tree2.handle)
            if n_:
                probe2[key] = ms_ / n_
        dom2 = max(probe2, key=probe2.get)
        zha.zha_profile_start(tree2.handle, dom2)
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        for s_ in range(args.warmup, args.warmup + steps):
            step2(s_)
        torch.cuda.synchronize()
        wall2 = time.perf_counter() - t2
        d2_ms, d2_n = zha.zha_profile_stop(tree2.handle)
        st2 = stats2.cpu().numpy()[args.warmup:args.warmup + steps]
        per2 = np.array([node_bytes(w2, L - row, key_form) for row in range(L)], dtype=np.float64)
        step2_b = float(np.mean((st2[:, :L, :].sum(axis=2) * per2[None, :]).sum(axis=1) +
                                st2[:, L, :].sum(axis=1) * w.block * 2 * d * 2))
        alg2 = float(np.mean([kernel_bytes(dom2, w2, st2[i], n0 + args.warmup + i + 1, key_form) for i in range(steps)]))
        ach2 = alg2 / (d2_ms / max(d2_n, 1) * 1e-3) / 1e9
        quant[fmt] = {
            "route": "frontier" if tree2.route_mode == 1 else "keys",
            "ms_per_step": round(wall2 * 1e3 / steps, 4), "queries_per_s": round(steps / wall2, 2),
            "speedup_vs_main_line": round(ms_per_step / (wall2 * 1e3 / steps), 3),
            "build_ms": round(min(b_ms), 4),
            "decode_step_alg_bytes": round(step2_b),
            "roofline": dict(bound="hbm", kernel=dom2, achieved=round(ach2, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                             frac=round(ach2 / HBM_PEAK_GBS, 4), avg_launch_ms=round(d2_ms / max(d2_n, 1), 4),
                             algorithmic_bytes_per_launch=round(alg2),
                             traffic=traffic_for(dom2, f"{w.name}_{fmt}planes")),
            "kernel_ms": {k: round(v, 4) for k, v in sorted(probe2.items(), key=lambda x: -x[1])},
        }
        log(f"[bench] {fmt} router planes ({quant[fmt]['route']}): {quant[fmt]['ms_per_step']:.3f} ms/step, "
            f"{quant[fmt]['queries_per_s']:.1f} queries/s; {dom2} {d2_ms / max(d2_n, 1):.4f} ms/launch "
            f"({ach2 / HBM_PEAK_GBS:.3f} of HBM)")
        tree2.close()
        del tree2

    # ---- multi-token append: a tree over N0 - m tokens grows by m rows at once (the rows
    # already hold their values, so the copy rewrites them unchanged)
    append_n = None
    m_app = args.append_chunk
    if m_app > 0 and n0 > m_app:
        tree3 = zha.Tree(cfg)
        Kc, Vc = Kd[:, n0 - m_app:n0].contiguous(), Vd[:, n0 - m_app:n0].contiguous()
        an_ms = []
        for _ in range(3):
            tree3.build(Kd, Vd, n0 - m_app, Rd)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            tree3.append_n(Kc, Vc)
            e1.record()
            torch.cuda.synchronize()
            an_ms.append(e0.elapsed_time(e1))
        am = float(np.median(an_ms))
        append_n = {"tokens": m_app, "onto_tokens": n0 - m_app, "ms": round(am, 4),
                    "tokens_per_s": round(m_app / (am * 1e-3)),
                    "single_append_ms": round(probe_ms.get("append", float("nan")), 4)}
        log(f"[bench] append_n of {m_app} tokens onto {n0 - m_app}: {am:.3f} ms "
            f"({m_app / (am * 1e-3) / 1e6:.1f} M tok/s; one-token append {probe_ms.get('append', float('nan')):.4f} ms)")
        # causal multi-query prefill of the last 64 tokens: per token, then batched
        per_token, batched = prefill_legs(zha, tree3, w, Kd, Vd, Qd, Rd, n0, min(64, total), (8, 16, 32, 64), dev)
        append_n["prefill"] = per_token
        append_n["prefill_batched"] = batched
        tree3.close()
        del tree3, Kc, Vc

    # stream-read probe: practical HBM read bandwidth of a plain streaming kernel (2 GiB)
    sst = torch.cuda.current_stream().cuda_stream
    nb = 1 << 31
    buf = torch.empty(nb, dtype=torch.uint8, device=dev)
    sink = torch.empty(4096, dtype=torch.int32, device=dev)
    best = 0.0
    for blocks in (256, 512, 1024, 2048, 4096):
        plib.zha_probe_stream_read(buf.data_ptr(), nb, sink.data_ptr(), blocks, sst)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            plib.zha_probe_stream_read(buf.data_ptr(), nb, sink.data_ptr(), blocks, sst)
        e1.record()
        torch.cuda.synchronize()
        best = max(best, nb * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    read_gbs = best
    log(f"[bench] stream-read probe {read_gbs:.0f} GB/s")
    if args.calib_copy:
        dst = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        plib.zha_probe_copy(buf.data_ptr(), dst.data_ptr(), 1 << 30, 2048, sst)
        torch.cuda.synchronize()
        del dst
    del buf

    cpu = None
    if not args.no_cpu:
        t = time.perf_counter()
        K0 = Kd[:1].float().cpu().numpy()
        V0 = Vd[:1].float().cpu().numpy()
        cpu = cpu_baseline(w, K0, V0, refs, queries, n0, args.cpu_budget)
        log(f"[bench] cpu baseline {cpu['value']:.4f} queries/s ({time.perf_counter() - t:.1f}s)")
        if w.n_tokens <= (1 << 20):
            t = time.perf_counter()
            cpu["all_cores"] = cpu_baseline_all_cores(w, n0, args.cpu_budget, total)
            log(f"[bench] cpu baseline, {cpu['all_cores']['cores']} processes: {cpu['all_cores']['value']:.4f} "
                f"queries/s ({time.perf_counter() - t:.1f}s)")

    rec = {
        "metric": METRIC,
        "value": round(qps, 2),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16+f32",
        "data": "synthetic",
        "config": {"workload": f"{w.name}_{n0}" + ("" if w.planes == "f32" else f"_{w.planes}planes") + ("_plevels" if p_levels else ""), "kv_tokens": n0, "head_dim": d, "q_heads": w.num_q_heads,
                   "kv_heads": w.num_kv_heads, "block": w.block, "levels": L, "num_ref": R, "top_p": w.top_p,
                   "router_planes": w.planes,
                   "top_p_levels": [round(x, 6) for x in p_levels] if p_levels else None,
                   "batch": 1, "layers": 1, "step": "append + decode"},
        "roofline": roofline,
        "roofline_step": roofline_step,
        "roofline_kernels": kernel_roofline,
        "cpu_baseline": cpu,
        "cold": cold,
        "cold_after_write": cold_write,
        "decode_step": {"route": "keys" if allkeys else "frontier", "level1_key_form": key_form, "alg_bytes": round(step_bytes), "achieved_GBps": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
                        "router_bytes": round(float(np.mean(router_b))), "gather_bytes": round(float(np.mean(gather_b))),
                        "frontier_union_per_level": timed_stats[:, :L, :].sum(axis=2).mean(axis=0).round(1).tolist(),
                        "kept_blocks_union": float(timed_stats[:, L, :].sum(axis=1).mean()),
                        # per KV head (levels 1..L, then the kept blocks): a head's grid share is
                        # fixed, so the largest sets the launch time
                        "union_per_kv_head": timed_stats.mean(axis=0).round(1).tolist()},
        "build": {"ms": round(build_s * 1e3, 4), "tokens_per_s": round(build_tok_s), "alg_bytes": round(build_bytes),
                  "frac_hbm": round(build_bytes / build_s / 1e9 / HBM_PEAK_GBS, 4)},
        "dense": {"ms": round(dense_ms, 4), "queries_per_s": round(1e3 / dense_ms, 2),
                  "kernel_ms": round(dense_ms_k / max(dense_n, 1), 4), "alg_bytes": dense_bytes,
                  "frac_hbm": round(dense_bytes / (dense_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                  "zha_speedup": round(dense_ms / ms_per_step, 3)},
        "frontier_route_f32_planes": quant.get("f32"),
        "bf16_router_planes": quant.get("bf16"),
        "fp4_router_planes": quant.get("fp4"),
        "append_n": append_n,
        "modeled_reference": MODELED_REFERENCE,
        "hbm_read_probe_GBps": round(read_gbs, 1),
        "kernel_ms": {k: round(v, 4) for k, v in sorted(probe_ms.items(), key=lambda x: -x[1])},
        "src_sha": src_sha(),
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
