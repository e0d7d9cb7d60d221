"""Summaries of rocprofv3 output for the ZHA decode path (CSV output, run on any host).

    python -m hierarchical_tree_indexed_03_amd.prof_summary trace DIR WORKLOAD --cmd "..." [--out FILE]
    python -m hierarchical_tree_indexed_03_amd.prof_summary pmc FETCH_DIR WRITE_DIR WORKLOAD --cmd "..." [--out FILE]
    python -m hierarchical_tree_indexed_03_amd.prof_summary mfma DIR WORKLOAD --trace TRACE_DIR --cmd "..." [--out FILE]
    python -m hierarchical_tree_indexed_03_amd.prof_summary stats DIR --prefix fit_,build_ --title "..." --cmd "..." [--out FILE]
        [--fetch FETCH_DIR --write WRITE_DIR --fetch-scale 2.0 --write-scale 1.0]

``trace`` reads ``*_kernel_trace.csv`` (``rocprofv3 --kernel-trace --stats --output-format csv``)
and attributes every dispatch of a decode (route_prep ... combine) to its router level: the
general-path launches of a decode run from the highest general level down to level 1, so
they are numbered from the end.  It prints a markdown table of per-level averages.

``pmc`` reads two ``*_counter_collection.csv`` files (one run with ``--pmc FETCH_SIZE``, one with
``--pmc WRITE_SIZE``), scales the counters by what they read for the plain 1 GiB copy kernel
of the probe library (bench.py --calib-copy), and writes the measured HBM bytes per launch
of level-1 scoring and of the attention kernel to ``profiles/traffic_<WORKLOAD>.json``, keyed
by the hash of the sources of each kernel.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
from collections import defaultdict

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SHARED = ["common.hpp", "kernels.hpp", "route_util.hpp"]
KERNEL_SRC = {
    "route_score": ["score.hip"],
    "route_select": ["select.hip"],
    "route_expand": ["expand.hip"],
    "attend": ["attend.hip"],
    "dense_attend": ["attend.hip"],
    "route_score.keys": ["allkeys.hip"],
    "route_select.keys": ["topdown.hip"],
    "append": ["build.hip"],
    "build": ["build.hip"],
}
CALIB_BYTES = 1 << 30


def kernel_sha(key: str) -> str:
    """Hash of the sources that define the kernels behind a profile key (plus shared headers)."""
    files = KERNEL_SRC.get(key) or KERNEL_SRC.get(key.split(".")[0])
    if files is None:
        files = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".hpp")))
    h = hashlib.sha256()
    for f in sorted(set(files) | set(SHARED)):
        p = os.path.join(CSRC, f)
        if os.path.exists(p):
            with open(p, "rb") as fh:
                h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def short(name: str) -> str:
    n = name.replace("zha::", "").replace("(anonymous namespace)::", "")
    return n.split("(")[0].replace("void ", "")


STAGE = {
    "route_score_kernel": "score", "route_score_keys_kernel": "score", "route_score_bf16_kernel": "score",
    "route_score_bf16_rows_kernel": "score", "route_hist_kernel": "hist",
    "route_bound_kernel": "bound", "route_classify_kernel": "classify", "route_resolve_kernel": "resolve",
    "route_expand_count_kernel": "expand_count", "route_expand_emit_kernel": "expand_emit",
}
SCORES = ("route_score_kernel", "route_score_keys_kernel", "route_score_bf16_kernel", "route_score_bf16_rows_kernel")


def decodes(rows):
    """Splits time-ordered dispatches into decodes: lists from route_prep (or, on the keys
    route, which launches no prep, from its scoring) to combine."""
    out, cur = [], None
    for r in rows:
        n = short(r["name"])
        if n.startswith("route_prep_kernel") or (n.startswith("route_score_allkeys_kernel") and cur is None):
            cur = [r]
        elif cur is not None:
            cur.append(r)
            if n.startswith("combine_kernel"):
                out.append(cur)
                cur = None
    return out


def label(dec):
    """(label, row) per dispatch of one decode.  The top levels (scored whole, selected
    top-down) are labelled .top; each general level starts with its score launch and the
    general levels are numbered from level 1 (the last one)."""
    names = [short(r["name"]).split("<")[0] for r in dec]
    top_score = {i - 1 for i, n in enumerate(names) if n == "route_topdown_kernel" and i > 0 and names[i - 1] in SCORES}
    general = [i for i, n in enumerate(names) if n in SCORES and i not in top_score]
    res = []
    lv = "top"
    for i, (n, r) in enumerate(zip(names, dec)):
        if i in top_score:
            res.append(("score.top", r))
            lv = "top"
            continue
        if n in SCORES:
            lv = f"l{len(general) - general.index(i)}"
        if n == "route_score_allkeys_kernel":
            res.append(("score.keys", r))
        elif n == "route_topdown_keys_kernel":
            res.append(("select.keys", r))
        elif n == "route_topdown_kernel":
            res.append(("select.top", r))
        elif n == "route_topdown_union_kernel":
            res.append(("union.top", r))
        elif n in STAGE:
            res.append((f"{STAGE[n]}.{lv}", r))
        else:
            res.append((n.replace("_kernel", ""), r))
    return res


def read_trace(d):
    files = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        sys.exit(f"no kernel_trace.csv under {d}")
    rows = []
    for f in files:
        for r in csv.DictReader(open(f)):
            rows.append(dict(name=r["Kernel_Name"], t0=int(r["Start_Timestamp"]), t1=int(r["End_Timestamp"]),
                             gz=int(r.get("Grid_Size_Z", 1) or 1),
                             grid=int(r.get("Grid_Size_X", 0) or 0) // max(1, int(r.get("Workgroup_Size_X", 1) or 1))))
    rows.sort(key=lambda r: r["t0"])
    return rows, files


def cmd_trace(a):
    rows, files = read_trace(a.dir)
    decs = decodes(rows)
    # the ZHA decodes are those whose attention is the routed (non-dense) kernel
    decs = [d for d in decs if any("attend_kernel" in r["name"] and "false" in r["name"] for r in d)]
    per = defaultdict(list)
    step_us = []
    for d in decs:
        for lab, r in label(d):
            per[lab].append((r["t1"] - r["t0"]) / 1e3)
        step_us.append((d[-1]["t1"] - d[0]["t0"]) / 1e3)
    order = sorted(per, key=lambda k: -sum(per[k]) / len(per[k]))
    lines = [f"# rocprofv3 kernel trace: ZHA decode, workload `{a.workload}`", "",
             "Command (from the repository root on the GPU host):", "", "```", a.cmd, "```", "",
             "Summarised with:", "", "```",
             f"python -m hierarchical_tree_indexed_03_amd.prof_summary trace {a.dir} {a.workload} --cmd '...'",
             "```", "",
             f"{len(decs)} routed decodes; decode span (first routing launch start to combine end) "
             f"avg {sum(step_us) / max(1, len(step_us)):.1f} us.  Per-level kernels are numbered from level 1 "
             "(the last general level of each decode).", "",
             "| launch | calls | avg us | min us | max us | share of decode |", "|---|---:|---:|---:|---:|---:|"]
    tot = sum(sum(v) / len(decs) for v in per.values()) if decs else 1.0
    for k in order:
        v = per[k]
        lines.append(f"| {k} | {len(v)} | {sum(v) / len(v):.1f} | {min(v):.1f} | {max(v):.1f} | "
                     f"{100 * sum(v) / len(decs) / tot:.1f}% |")
    stats = glob.glob(os.path.join(a.dir, "**", "*kernel_stats.csv"), recursive=True)
    if stats:
        lines += ["", "rocprofv3 --stats (all dispatches of the run, top 15):", "",
                  "| kernel | calls | avg us | min us | max us |", "|---|---:|---:|---:|---:|"]
        for r in list(csv.DictReader(open(stats[0])))[:15]:
            lines.append(f"| {short(r['Name'])[:60]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                         f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} |")
    text = "\n".join(lines) + "\n"
    if a.out:
        with open(a.out, "w") as f:
            f.write(text)
    print(text)


def cmd_stats(a):
    """Per-kernel totals of a rocprofv3 --stats run, restricted to kernels whose short name
    starts with one of a.prefix (comma separated)."""
    stats = glob.glob(os.path.join(a.dir, "**", "*kernel_stats.csv"), recursive=True)
    if not stats:
        sys.exit(f"no kernel_stats.csv under {a.dir}")
    pre = tuple(p for p in a.prefix.split(",") if p)
    rows = [r for r in csv.DictReader(open(stats[0])) if short(r["Name"]).startswith(pre)]
    total = sum(float(r["TotalDurationNs"]) for r in rows) or 1.0
    lines = [f"# rocprofv3 kernel statistics: {a.title}", "", "Command (from the repository root on the GPU host):",
             "", "```", a.cmd, "```", "", "Summarised with:", "", "```",
             f"python -m hierarchical_tree_indexed_03_amd.prof_summary stats <dir> --prefix {a.prefix} --title '...' --cmd '...'",
             "```", "", "| kernel | calls | avg us | min us | max us | share of these kernels |",
             "|---|---:|---:|---:|---:|---:|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        lines.append(f"| {short(r['Name'])[:70]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{100 * float(r['TotalDurationNs']) / total:.1f}% |")
    if a.fetch and a.write:
        # measured HBM bytes per dispatch: FETCH_SIZE and WRITE_SIZE (KiB) times the scale the
        # same counters need on the plain 1 GiB copy kernel
        per = defaultdict(lambda: [[], []])
        for i, (d, c) in enumerate(((a.fetch, "FETCH_SIZE"), (a.write, "WRITE_SIZE"))):
            for r in read_pmc(d, c):
                if short(r["name"]).startswith(pre):
                    per[short(r["name"])][i].append(r["v"])
        lines += ["", f"Measured HBM traffic per dispatch (FETCH_SIZE x {a.fetch_scale}, WRITE_SIZE x "
                      f"{a.write_scale}, the copy-kernel calibration):", "",
                  "| kernel | dispatches | read MB | written MB |", "|---|---:|---:|---:|"]
        for k in sorted(per, key=lambda k: -sum(per[k][0]) / max(1, len(per[k][0]))):
            fv, wv = per[k]
            if fv and wv:
                lines.append(f"| {k[:70]} | {len(fv)} | {sum(fv) / len(fv) * 1024 * a.fetch_scale / 1e6:.1f} | "
                             f"{sum(wv) / len(wv) * 1024 * a.write_scale / 1e6:.1f} |")
    text = "\n".join(lines) + "\n"
    if a.out:
        with open(a.out, "w") as f:
            f.write(text)
    print(text)


def read_pmc(d, counter):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        sys.exit(f"no counter_collection.csv under {d}")
    disp = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            k = int(r["Dispatch_Id"])
            e = disp.setdefault(k, dict(name=r["Kernel_Name"], v=0.0,
                                        gz=int(r.get("Grid_Size_Z", 1) or 1) if "Grid_Size_Z" in r else 1))
            e["v"] += float(r["Counter_Value"])
    return [dict(id=k, **disp[k]) for k in sorted(disp)]


def pmc_groups(rows):
    """Calibration copy values and, per labelled launch of the routed decodes (score.top,
    score.l1, attend, ...), the counter values of its dispatches."""
    calib = [r["v"] for r in rows if short(r["name"]) == "copy_kernel"]
    per = defaultdict(list)
    for d in decodes(rows):
        if not any("attend_kernel" in r["name"] and "false" in r["name"] for r in d):
            continue
        for lab, r in label(d):
            per[lab].append(r["v"])
    return calib, per


def cmd_pmc(a):
    fetch = read_pmc(a.fetch_dir, "FETCH_SIZE")
    write = read_pmc(a.write_dir, "WRITE_SIZE")
    cf, fper = pmc_groups(fetch)
    cw, wper = pmc_groups(write)
    if not cf or not cw:
        sys.exit("calibration copy kernel not found (run bench.py with --calib-copy)")
    # counters are in KiB; scale each so the 1 GiB copy reads 1 GiB and writes 1 GiB
    kf = CALIB_BYTES / (cf[-1] * 1024.0)
    kw = CALIB_BYTES / (cw[-1] * 1024.0)
    mean = lambda v: sum(v) / len(v) if v else None
    out = {"workload": a.workload, "calib": {"copy_bytes": CALIB_BYTES, "fetch_kib": cf[-1], "write_kib": cw[-1],
                                             "fetch_scale": kf, "write_scale": kw},
           "command": a.cmd, "kernels": {}}
    keymap = {"score.top": "route_score.top", "score.l1": "route_score.l1", "score.l2": "route_score.l2",
              "score.keys": "route_score.keys", "select.keys": "route_select.keys", "attend": "attend"}
    for lab, key in keymap.items():
        fv, wv = fper.get(lab), wper.get(lab)
        if fv and wv:
            fb, wb = mean(fv) * 1024 * kf, mean(wv) * 1024 * kw
            out["kernels"][key] = {"src_sha": kernel_sha(key), "bytes": round(fb + wb), "fetch_bytes": round(fb),
                                   "write_bytes": round(wb), "launches": [len(fv), len(wv)]}
    path = a.out or os.path.join(ROOT, "profiles", f"traffic_{a.workload}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
                 "SQ_INSTS_VALU_MFMA_MOPS_F32", "SQ_BUSY_CU_CYCLES")
SIMD_NUM = 256 * 4           # MI355X: 256 compute units x 4 SIMDs
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}


def cmd_mfma(a):
    """MFMA use of the build kernels from one counter run (MFMA_COUNTERS), with the kernel
    durations of a kernel trace of the same workload (the counter run's own timestamps include
    the collection).  Dispatches of one kernel are averaged."""
    files = glob.glob(os.path.join(a.dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        sys.exit(f"no counter_collection.csv under {a.dir}")
    disp = defaultdict(lambda: defaultdict(list))
    names = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            k = int(r["Dispatch_Id"])
            disp[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
            names[k] = short(r["Kernel_Name"])
    dur = defaultdict(list)
    if a.trace:
        rows, _ = read_trace(a.trace)
        for r in rows:
            dur[short(r["name"])].append((r["t1"] - r["t0"]) / 1e3)
    per = defaultdict(list)       # kernel -> [(util %, bf16 GFLOP, f32 GFLOP)] per dispatch
    for k in sorted(disp):
        n = names[k]
        if not (n.startswith("build_") or n.startswith("quantise_")):
            continue
        v = disp[k]
        busy = sum(v["SQ_VALU_MFMA_BUSY_CYCLES"])
        grbm = max(v["GRBM_GUI_ACTIVE"]) if v["GRBM_GUI_ACTIVE"] else 0.0
        per[n].append((100.0 * busy / (grbm * SIMD_NUM) if grbm else 0.0,
                       sum(v["SQ_INSTS_VALU_MFMA_MOPS_BF16"]) * 512 / 1e9,
                       sum(v["SQ_INSTS_VALU_MFMA_MOPS_F32"]) * 512 / 1e9))
    lines = [f"# MFMA use of the tree build, workload `{a.workload}`", "",
             "Counter run (from the repository root on the GPU host):", "", "```", a.cmd, "```", "",
             "Durations come from the kernel trace of the same workload"
             + (f" (`{a.trace_cmd}`)" if a.trace_cmd else "") + ".", "",
             "Summarised with:", "", "```",
             f"python -m hierarchical_tree_indexed_03_amd.prof_summary mfma {a.dir} "
             f"{a.workload} --trace {a.trace} --cmd '...' --trace-cmd '...'",
             "```", "",
             "MFMA utilisation = SQ_VALU_MFMA_BUSY_CYCLES summed over the chip / (GRBM_GUI_ACTIVE x "
             "1,024 SIMDs), the MfmaUtil expression of rocprofv3; MFMA flops = MOPS x 512.", "",
             "| kernel | dispatches | MFMA util | bf16 MFMA GFLOP | f32 MFMA GFLOP | avg duration us "
             "| bf16 TFLOP/s (of 2,500) | f32 TFLOP/s (of 157.3) |",
             "|---|---:|---:|---:|---:|---:|---:|---:|"]
    for n, xs in per.items():
        m = len(xs)
        util, fb, ff = (sum(x[i] for x in xs) / m for i in range(3))
        ds = dur.get(n)
        d_us = sum(ds) / len(ds) if ds else float("nan")
        lines.append(f"| {n[:60]} | {m} | {util:.1f}% | {fb:.2f} | {ff:.2f} | {d_us:.1f} | "
                     f"{fb / d_us * 1e3:.1f} | {ff / d_us * 1e3:.1f} |")
    text = "\n".join(lines) + "\n"
    if a.out:
        with open(a.out, "w") as f:
            f.write(text)
    print(text)


def main():
    ap = argparse.ArgumentParser()
    sp = ap.add_subparsers(dest="mode", required=True)
    t = sp.add_parser("trace")
    t.add_argument("dir")
    t.add_argument("workload")
    t.add_argument("--cmd", default="")
    t.add_argument("--out", default=None)
    p = sp.add_parser("pmc")
    p.add_argument("fetch_dir")
    p.add_argument("write_dir")
    p.add_argument("workload")
    p.add_argument("--cmd", default="")
    p.add_argument("--out", default=None)
    m = sp.add_parser("mfma")
    m.add_argument("dir")
    m.add_argument("workload")
    m.add_argument("--trace", default=None)
    m.add_argument("--cmd", default="")
    m.add_argument("--trace-cmd", default="")
    m.add_argument("--out", default=None)
    x = sp.add_parser("stats")
    x.add_argument("dir")
    x.add_argument("--prefix", default="")
    x.add_argument("--title", default="")
    x.add_argument("--cmd", default="")
    x.add_argument("--out", default=None)
    x.add_argument("--fetch", default=None, help="directory of a --pmc FETCH_SIZE run")
    x.add_argument("--write", default=None, help="directory of a --pmc WRITE_SIZE run")
    x.add_argument("--fetch-scale", type=float, default=2.0)
    x.add_argument("--write-scale", type=float, default=1.0)
    a = ap.parse_args()
    {"trace": cmd_trace, "pmc": cmd_pmc, "mfma": cmd_mfma, "stats": cmd_stats}[a.mode](a)


if __name__ == "__main__":
    main()
