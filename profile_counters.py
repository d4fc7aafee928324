"""Hardware-counter summaries of the hot path's kernels, taken with rocprofv3 on an MI355X.

    python profile_counters.py hbm  [--config 4] [--out DIR]   # FETCH_SIZE / WRITE_SIZE
    python profile_counters.py mfma [--config 3] [--out DIR]   # MFMA busy cycles and ops
    python profile_counters.py balance [--config 6] [--out DIR] # CU busy fraction, occupancy
    python profile_counters.py timeline [--config 4] [--out DIR] [--bench-args ...]
                                                              # per-workgroup phase stamps

Each counter pass is its own `rocprofv3 --pmc ... -- python3 bench.py ...` child process (the
profiler's library must start with the program, so this script never touches the GPU
itself), run from /tmp with TMPDIR=/tmp and a time limit.

hbm: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of every kernel of the step, each scaled by
what the same counter reads for a plain 256 MiB device-to-device copy of known size, give HBM
bytes per launch of the indexer call and of the attention call (its kernels summed).  The
result goes to profiles/decode_counters.json, tied to the kernel sources by the digest
bench.py computes (bench.py reports `traffic` only while it matches), and a Markdown table is
printed.

mfma: SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE and SQ_INSTS_VALU_MFMA_MOPS_BF16 per
dispatch.  Utilisation = busy cycles / (GUI-active cycles x 1024 SIMDs), the profiler's own
MfmaUtil definition; flops = MOPS x 512; the durations come from a kernel-trace pass of the
same command.  A Markdown table is printed.

balance: the profiler's derived SIMD_UTILIZATION (summed SQ_BUSY_CU_CYCLES over the clock count
and the CU count), OccupancyPercent and MeanOccupancyPerActiveCU per dispatch, with the
durations of a kernel-trace pass, for the natural query order and for bench.py's zigzag order
(4-query tiles paired head and tail).  A kernel whose work is spread evenly keeps its CUs busy
to its end; CUs left idle while a few long workgroups finish would show as a low busy fraction.

timeline: no profiler.  bench.py --timeline runs the step with the measurement build of the
library (libdsa_timeline.so, `python -m sparse_indexed_attention_amd.build --timeline`), whose
kernels stamp the constant 100 MHz clock at the end of each phase of every workgroup
(include/dsa_timeline.h), for 20 recorded steps.  The summary gives, in microseconds from the
step's first indexer workgroup start, when the phases end across workgroups (median, 90th
percentile, latest, each the median over the recorded steps) and how long the merges' phases
take.  The stamps add a store per phase and workgroup; the library's own timing is taken
without them.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import subprocess
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.abspath(__file__))
SIMDS = 256 * 4


def run_prof(out_dir, tag, prof_args, bench_args, limit=240):
    d = os.path.join(out_dir, tag)
    cmd = ["rocprofv3", *prof_args, "--output-format", "csv", "-d", d, "-o", tag, "--",
           sys.executable, os.path.join(ROOT, "bench.py"), *bench_args]
    print("profile_counters: " + " ".join(cmd), flush=True)
    env = dict(os.environ, TMPDIR="/tmp")
    r = subprocess.run(["timeout", "-s", "KILL", str(limit), *cmd], cwd="/tmp", env=env)
    if r.returncode != 0:
        # rocprofv3 may end with a segmentation fault after a complete run; the caller checks
        # that the result files exist
        print(f"profile_counters: {tag} exited {r.returncode}", flush=True)
    return d, " ".join(cmd[:cmd.index("-d")] + cmd[cmd.index("--"):]).replace(ROOT, "$ROOT")


def read_csv(d, suffix):
    files = glob.glob(os.path.join(d, "**", f"*{suffix}.csv"), recursive=True)
    if not files:
        raise SystemExit(f"profile_counters: no *{suffix}.csv under {d}")
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            rows += list(csv.DictReader(fh))
    return rows


def short(name):
    n = name.replace("(anonymous namespace)::", "").replace("dsa::", "").strip()
    if n.startswith("void "):
        n = n[5:]
    return n.split("(")[0].strip()


def counters_per_kernel(d):
    """{kernel: {counter: mean value per dispatch}} from a --pmc pass."""
    acc = defaultdict(lambda: defaultdict(float))
    disp = defaultdict(set)
    for r in read_csv(d, "counter_collection"):
        k = short(r["Kernel_Name"])
        acc[k][r["Counter_Name"]] += float(r["Counter_Value"])
        disp[k].add(r["Dispatch_Id"])
    return {k: {c: v / len(disp[k]) for c, v in cs.items()} for k, cs in acc.items()}, \
        {k: len(v) for k, v in disp.items()}


def durations(d):
    """{kernel: (calls, mean us)} from a --kernel-trace pass."""
    acc = defaultdict(list)
    for r in read_csv(d, "kernel_trace"):
        acc[short(r["Kernel_Name"])].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return {k: (len(v), sum(v) / len(v)) for k, v in acc.items()}


def call_of(kernel):
    if kernel.startswith("indexer_topk_kernel"):
        return "indexer"
    if kernel.startswith("sfa_"):
        return "sparse_attn"
    return None


def hbm(args):
    sys.path.insert(0, ROOT)
    import bench
    ba = ["--steps", "3", "--warmup", "1", "--no-cpu-baseline", "--config", str(args.config)]
    cmds, res = [], {}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        d, c = run_prof(args.out, f"pmc_{ctr.lower()}", ["--pmc", ctr], ba)
        res[ctr], n = counters_per_kernel(d)
        cmds.append(c)
        d, c = run_prof(args.out, f"pmc_copy_{ctr.lower()}", ["--pmc", ctr], ["--calibrate-copy", "256"])
        cal, _ = counters_per_kernel(d)
        cmds.append(c)
        copy_k = [k for k in cal if "copy" in k.lower()]
        res["copy_" + ctr] = cal[copy_k[0]][ctr]
    moved_kib = 256 * 1024.0
    ff = moved_kib / res["copy_FETCH_SIZE"]
    wf = moved_kib / res["copy_WRITE_SIZE"]
    kernels = sorted(k for k in res["FETCH_SIZE"] if call_of(k))
    calls = {}
    table = ["| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled read MB | scaled write MB |",
             "|---|---:|---:|---:|---:|"]
    for k in kernels:
        f = res["FETCH_SIZE"][k]["FETCH_SIZE"]
        w = res["WRITE_SIZE"].get(k, {}).get("WRITE_SIZE", 0.0)
        rb, wb = f * 1024 * ff, w * 1024 * wf
        table.append(f"| `{k}` | {f:.0f} | {w:.0f} | {rb / 1e6:.1f} | {wb / 1e6:.1f} |")
        e = calls.setdefault(call_of(k), {"kernels": [], "hbm_bytes_per_launch": 0.0,
                                          "read_bytes": 0.0, "write_bytes": 0.0})
        e["kernels"].append(k)
        e["hbm_bytes_per_launch"] += rb + wb
        e["read_bytes"] += rb
        e["write_bytes"] += wb
    out = {"workload": bench_workload(args.config), "source_digest": bench.source_digest(),
           "calls": calls,
           "calibration": {"kernel": "device-to-device copy (bench.py --calibrate-copy 256)",
                           "bytes": 256 << 20, "fetch_kib": res["copy_FETCH_SIZE"],
                           "write_kib": res["copy_WRITE_SIZE"], "fetch_factor": ff,
                           "write_factor": wf},
           "commands": cmds}
    path = os.path.join(ROOT, "profiles", "decode_counters.json") if args.write else \
        os.path.join(args.out, "decode_counters.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(f"profile_counters: wrote {path}")
    print(f"copy calibration: fetch factor {ff:.3f}, write factor {wf:.3f}")
    print("\n".join(table))
    for c, e in calls.items():
        print(f"{c}: {e['hbm_bytes_per_launch'] / 1e6:.1f} MB per launch "
              f"(read {e['read_bytes'] / 1e6:.1f}, write {e['write_bytes'] / 1e6:.1f})")
    print("commands:\n" + "\n".join("    cd /tmp && export TMPDIR=/tmp && " + c for c in cmds))


def bench_workload(cfg):
    sys.path.insert(0, ROOT)
    from synth import workload
    return workload(cfg).name


def mfma(args):
    ba = ["--steps", "2", "--warmup", "1", "--no-cpu-baseline", "--config", str(args.config)]
    d, c1 = run_prof(args.out, "mfma_busy",
                     ["--pmc", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "SQ_INSTS_VALU_MFMA_MOPS_BF16"], ba, 600)
    ctr, n = counters_per_kernel(d)
    d, c2 = run_prof(args.out, "mfma_util", ["--pmc", "MfmaUtil"], ba, 600)
    util_d, _ = counters_per_kernel(d)
    d, c3 = run_prof(args.out, "mfma_trace", ["--kernel-trace"], ba, 600)
    dur = durations(d)
    print(f"workload {bench_workload(args.config)}")
    print("| kernel | dispatches | mean us | MfmaUtil % | busy / (GUI x 1024) | bf16 MFMA TFLOP/s (MOPS x 512 / time) | of 2500 |")
    print("|---|---:|---:|---:|---:|---:|---:|")
    for k in sorted(ctr):
        if not call_of(k):
            continue
        cs = ctr[k]
        raw = cs["SQ_VALU_MFMA_BUSY_CYCLES"] / (cs["GRBM_GUI_ACTIVE"] * SIMDS) if cs.get("GRBM_GUI_ACTIVE") else float("nan")
        mu = util_d.get(k, {}).get("MfmaUtil", float("nan"))
        flops = cs.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * 512
        us = dur.get(k, (0, float("nan")))[1]
        tf = flops / (us * 1e-6) / 1e12 if us == us and us > 0 else float("nan")
        print(f"| `{k}` | {n[k]} | {us:.1f} | {mu:.1f} | {raw:.3f} | {tf:.0f} | {tf / 2500:.3f} |")
        print(f"<!-- {k}: busy {cs['SQ_VALU_MFMA_BUSY_CYCLES']:.4g}, gui {cs['GRBM_GUI_ACTIVE']:.4g}, "
              f"mops_bf16 {cs.get('SQ_INSTS_VALU_MFMA_MOPS_BF16', 0):.4g} -->")
    print("commands:\n" + "\n".join("    cd /tmp && export TMPDIR=/tmp && " + c for c in (c1, c2, c3)))


def balance(args):
    rows, cmds = [], []
    for order in ("natural", "zigzag"):
        ba = ["--steps", "2", "--warmup", "1", "--no-cpu-baseline", "--config", str(args.config),
              "--order", order]
        d, c1 = run_prof(args.out, f"balance_{order}",
                         ["--pmc", "SIMD_UTILIZATION", "OccupancyPercent", "MeanOccupancyPerActiveCU"], ba, 600)
        ctr, n = counters_per_kernel(d)
        d, c2 = run_prof(args.out, f"balance_trace_{order}", ["--kernel-trace"], ba, 600)
        dur = durations(d)
        cmds += [c1, c2]
        for k in sorted(ctr):
            if call_of(k):
                cs = ctr[k]
                rows.append(f"| {order} | `{k}` | {n[k]} | {dur.get(k, (0, float('nan')))[1]:.1f} | "
                            f"{cs.get('SIMD_UTILIZATION', float('nan')):.3f} | "
                            f"{cs.get('OccupancyPercent', float('nan')):.1f} | "
                            f"{cs.get('MeanOccupancyPerActiveCU', float('nan')):.2f} |")
    print(f"workload {bench_workload(args.config)}")
    print("| query order | kernel | dispatches | mean us | SIMD_UTILIZATION | OccupancyPercent | MeanOccupancyPerActiveCU |")
    print("|---|---|---:|---:|---:|---:|---:|")
    print("\n".join(rows))
    print("commands:\n" + "\n".join("    cd /tmp && export TMPDIR=/tmp && " + c for c in cmds))


def _pct(xs, q):
    import numpy as np
    xs = [x for x in xs if x is not None]
    return float(np.percentile(xs, q)) if xs else float("nan")


def timeline(args):
    lib = os.path.join(ROOT, "sparse_indexed_attention_amd", "libdsa_timeline.so")
    if not os.path.exists(lib) and not args.from_json:
        raise SystemExit("profile_counters: build libdsa_timeline.so first "
                         "(python -m sparse_indexed_attention_amd.build --timeline)")
    path = args.from_json or os.path.join(args.out, f"timeline_config{args.config}.json")
    if args.from_json:
        with open(path) as f:
            return timeline_summary(json.load(f))
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--config", str(args.config),
           "--steps", "20", "--warmup", "5", "--no-cpu-baseline", "--timeline", path,
           *args.bench_args]
    print("profile_counters: DSA_LIB_PATH=$ROOT/sparse_indexed_attention_amd/libdsa_timeline.so "
          + " ".join(cmd).replace(ROOT, "$ROOT"), flush=True)
    r = subprocess.run(["timeout", "-k", "10", "240", *cmd], env=dict(os.environ, DSA_LIB_PATH=lib))
    if r.returncode != 0:
        raise SystemExit(f"profile_counters: bench.py --timeline exited {r.returncode}")
    with open(path) as f:
        timeline_summary(json.load(f))


def timeline_summary(data):
    import numpy as np
    steps = data["steps"]

    def per_step(fn):
        """median over the recorded steps of fn(step) (a number)"""
        return float(np.median([fn(s) for s in steps]))

    def col(s, kern, slot, only=None):
        return [v[slot] for v in s[kern].values() if v[slot] is not None and (only is None or only(v))]

    print(f"\n### Phase ends, {data['workload']} ({data['queries']} queries; {len(steps)} recorded "
          f"steps; µs from the first indexer workgroup's start)\n")
    print("| kernel | phase end | workgroups | median | p90 | latest |")
    print("|---|---|---|---|---|---|")
    rows = [("indexer", 0, "start", None), ("indexer", 1, "split scored", None),
            ("indexer", 2, "candidates stored", None), ("indexer", 3, "arrival counted", None),
            ("indexer", 4, "merge: headers read", None), ("indexer", 5, "merge: list staged", None),
            ("indexer", 6, "merge: K-th key found", None), ("indexer", 7, "merge: output written", None),
            ("attention", 0, "start", None), ("attention", 1, "pool rows resolved", None),
            ("attention", 2, "first tiles and query rows landed", None),
            ("attention", 3, "query fragments in registers", None),
            ("attention", 4, "last tile done", None), ("attention", 5, "outputs/partials written", None),
            ("combine", 0, "start", None), ("combine", 5, "written", None)]
    for kern, slot, name, only in rows:
        if not any(col(s, kern, slot) for s in steps):
            continue
        n = int(per_step(lambda s: len(col(s, kern, slot))))
        print(f"| {kern} | {name} | {n} | {per_step(lambda s: _pct(col(s, kern, slot), 50)):.2f} | "
              f"{per_step(lambda s: _pct(col(s, kern, slot), 90)):.2f} | "
              f"{per_step(lambda s: _pct(col(s, kern, slot), 100)):.2f} |")
    # a split's steps from scoring to arrival (finer stamps; absent in older records)
    def steps_of(pairs, kern, only=None):
        rows_ = []
        for name, a, b in pairs:
            ds = lambda s: [v[b] - v[a] for v in s[kern].values()
                            if len(v) > max(a, b) and v[a] is not None and v[b] is not None
                            and (only is None or only(v))]
            if any(ds(s) for s in steps):
                rows_.append(f"| {name} | {per_step(lambda s: _pct(ds(s), 50)):.2f} | "
                             f"{per_step(lambda s: _pct(ds(s), 90)):.2f} |")
        return rows_
    r_ = steps_of((("choosing the cut", 1, 16), ("issuing candidate and header stores", 16, 17),
                   ("draining the stores", 17, 2), ("counting the arrival", 2, 3)), "indexer")
    if r_:
        print("\n### A split from scored to arrived\n")
        print("| step | median µs | p90 µs |")
        print("|---|---|---|")
        print("\n".join(r_))
    # the merges: phase durations of the merging workgroups (one per query)
    merging = lambda v: v[15] == 1 and v[7] is not None
    if any(any(merging(v) for v in s["indexer"].values()) for s in steps):
        print("\n### Merges (the last-arriving split of each query)\n")
        print("| phase | median µs | max µs |")
        print("|---|---|---|")
        for name, a, b in (("arrival to headers read", 3, 4), ("staging the list", 4, 5),
                           ("finding the K-th key's bin", 5, 18), ("from the bin to the K-th key", 18, 6),
                           ("finding the K-th key", 5, 6), ("writing the output", 6, 7),
                           ("whole merge", 3, 7)):
            ds = lambda s: [v[b] - v[a] for v in s["indexer"].values()
                            if merging(v) and len(v) > max(a, b) and v[a] is not None and v[b] is not None]
            if not any(ds(s) for s in steps):
                continue
            print(f"| {name} | {per_step(lambda s: _pct(ds(s), 50)):.2f} | "
                  f"{per_step(lambda s: _pct(ds(s), 100)):.2f} |")
    print("\n### Main loops: wave 0's shader-clock cycles per step (s_memtime)\n")
    print("| kernel | loop | steps | waiting for loads | computing (with barriers) | issuing loads "
          "| wait share |")
    print("|---|---|---|---|---|---|---|")
    for kern, loop in (("indexer", "key groups (scoring)"),
                       ("attention", "tile pairs (64-head decode kernel) or tiles")):
        def cyc(s, slot):
            return [v[slot] / v[10] for v in s[kern].values() if v[10]]
        if not any(cyc(s, 8) for s in steps):
            continue
        w = per_step(lambda s: _pct(cyc(s, 8), 50))
        c = per_step(lambda s: _pct(cyc(s, 9), 50))
        n = per_step(lambda s: _pct([v[10] for v in s[kern].values() if v[10]], 50))
        has_i = any(len(v) > 19 and v[19] for s in steps for v in s[kern].values())
        i_ = per_step(lambda s: _pct([v[19] / v[10] for v in s[kern].values() if v[10]], 50)) if has_i else 0.0
        print(f"| {kern} | {loop} | {n:.0f} | {w:.0f} | {c:.0f} | "
              f"{f'{i_:.0f}' if has_i else '-'} | {w / (w + c + i_):.2f} |")
    # shader clock rate: s_memtime ticks over wall-clock µs between the two readings
    for kern, a, b in (("indexer", 0, 1), ("attention", 0, 4)):
        def mhz(s):
            return [(v[12] - v[11]) / (v[b] - v[a]) for v in s[kern].values()
                    if v[11] and v[12] and v[a] is not None and v[b] is not None and v[b] > v[a]]
        if any(mhz(s) for s in steps):
            print(f"\n{kern}: shader clock {per_step(lambda s: _pct(mhz(s), 50)):.0f} MHz (median over "
                  f"workgroups of s_memtime ticks per wall-clock µs)")
    loop0 = lambda s: [v[13] for v in s["indexer"].values() if v[13] is not None]
    if any(loop0(s) for s in steps):
        print(f"indexer: scoring loops start at {per_step(lambda s: _pct(loop0(s), 50)):.2f} µs (median), "
              f"{per_step(lambda s: _pct(loop0(s), 100)):.2f} µs (latest)")
    if any(s["attention"] for s in steps):
        print("\n### Attention workgroups: phase durations\n")
        print("| phase | median µs | p90 µs |")
        print("|---|---|---|")
        for name, a, b in (("start to rows resolved", 0, 1), ("rows resolved to first tiles landed", 1, 2),
                           ("query fragments to registers", 2, 3), ("tile loop", 3, 4),
                           ("start to last tile done", 0, 4),
                           ("writing", 4, 5), ("whole workgroup", 0, 5)):
            ds = lambda s: [v[b] - v[a] for v in s["attention"].values()
                            if v[a] is not None and v[b] is not None]
            if any(ds(s) for s in steps):
                print(f"| {name} | {per_step(lambda s: _pct(ds(s), 50)):.2f} | "
                      f"{per_step(lambda s: _pct(ds(s), 90)):.2f} |")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("mode", choices=("hbm", "mfma", "balance", "timeline"))
    ap.add_argument("--config", type=int, default=None)
    ap.add_argument("--out", default=os.path.join(ROOT, "gpurun_out", "counters"))
    ap.add_argument("--write", action="store_true",
                    help="hbm: write profiles/decode_counters.json (else into --out)")
    ap.add_argument("--from-json", default="", help="timeline: summarize a recorded file only")
    ap.add_argument("--bench-args", nargs=argparse.REMAINDER, default=[],
                    help="timeline: further bench.py arguments (e.g. --sfa-kv fp8)")
    args = ap.parse_args()
    if args.config is None:
        args.config = {"hbm": 4, "mfma": 3, "balance": 6, "timeline": 4}[args.mode]
    args.out = os.path.abspath(args.out)        # the profiler runs from /tmp
    os.makedirs(args.out, exist_ok=True)
    {"hbm": hbm, "mfma": mfma, "balance": balance, "timeline": timeline}[args.mode](args)


if __name__ == "__main__":
    main()
