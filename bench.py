"""Throughput of the DSA hot path (lightning indexer + Top-K + Sparse Flash Attention) on one
MI355X.

One step = dsa_indexer_topk then dsa_sparse_attn over one batch of decode queries, both on
the current stream, inputs resident in HBM.  Default workload: quantized decode at 128K
context (batch 8, per-sequence context uniform in [64K, 128K], fp8-e4m3 index keys with
per-token scales, bf16 queries, indexer 64 heads x 128, Top-K 2048, SFA 128 heads over the
576/512 latent cache in 64-token pages scattered by a random block table).

The working set of one step (~125 MB) fits the 256 MB Infinity Cache, so the timed loop
rotates over `--copies` independent device copies of all pools, tables and queries: a copy
is reused only after ~1 GB of other copies has been touched.

Prints one JSON line (see the keys below).  `value` is queries / second over exactly --steps
steps between two synchronizations.  After that region each call is timed alone: launched back
to back over the rotating copies behind a GPU sleep that keeps the queue full while the host
enqueues, with HIP events between batches of calls on the stream the library launches on
(samples, median, min, p10/p90 in the line).  The roofline of the dominant kernel (the
indexer, HBM-bound in decode) is its algorithmic bytes per launch / that mean call time; the
attention call gets its own.  `traffic` comes from the committed rocprofv3 counter summary
(profiles/decode_counters.json, written by profile_counters.py) while its source digest
matches the kernels.  The CPU oracle is timed on a bounded sample.

    python bench.py [--gpus 1] [--steps 200] [--warmup 10] [--config 4] [--sfa-kv fp8]
    python bench.py --config 6 --shards 4 [--layout zigzag|contiguous] --steps 5 --warmup 2

--sfa-kv fp8 stores the latent cache as fp8 rows quantized per 128-column tile (written by
dsa_store_kv on the GPU before timing) instead of bf16 rows.  --idx-keys mxfp8 stores the
index keys in MXFP8 (e4m3 codes, one E8M0 scale byte per group of 32 dims, written by
dsa_store_index_keys on the GPU from the same N(0,1) keys) instead of fp8 with per-token
scales; the CPU baseline then reads the oracle's quantization of the same keys.  --shards G
times a chunk of queries cut into G shards (zigzag head-tail pairs or contiguous ranges), each
shard's step on its own: the share one device of a context-parallel group would run.
"""
from __future__ import annotations

import argparse
import copy
import dataclasses
import hashlib
import re
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode queries/sec (indexer+TopK+SFA) at 128K ctx; % peak HBM BW / MFMA"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
ELEM = {"f32": 4, "bf16": 2, "fp8": 1, "mxfp8": 1}
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "decode_counters.json")


def indexer_bytes(spec, V):
    """Algorithmic bytes one indexer launch must move: every visible key (+ its fp8 scale),
    one block-table entry per 64-token page, the queries and head weights, the index list."""
    ek = ELEM[spec.k_dtype]
    sk = {"fp8": 4, "mxfp8": spec.idx_dim // 32}.get(spec.k_dtype, 0)
    eq = ELEM[spec.q_dtype]
    b = 0
    for v in V:
        v = int(v)
        b += v * (spec.idx_dim * ek + sk)
        if spec.block_size:
            b += 4 * math.ceil(v / spec.block_size)
        b += spec.idx_heads * (spec.idx_dim * eq + 4)
        b += 4 * spec.top_k
    return b


KV_FP8_ROW_BYTES = 656


def sfa_bytes(spec, V):
    """Algorithmic bytes of one SFA launch: the index list, the selected latent rows, the
    queries and the outputs (fp8 rows: 656 bytes, bf16 queries and outputs)."""
    fp8 = spec.kv_dtype == "fp8"
    e = 2 if fp8 else ELEM[spec.kv_dtype]
    row = KV_FP8_ROW_BYTES if fp8 else spec.d_qk * e
    b = 0
    for v in V:
        k_eff = min(spec.top_k, int(v))
        b += 4 * spec.top_k + k_eff * row
        b += spec.sfa_heads * (spec.d_qk * e + spec.d_v * e)
    return b


class Fp8RowsOfBf16Pool:
    """The oracle's fp8 rows of a bf16 latent pool, quantized when indexed (the CPU baseline
    reads only the selected rows of each query)."""

    def __init__(self, bf16_pool):
        self.pool = bf16_pool

    def __getitem__(self, rows):
        import oracle
        return oracle.quantize_kv_fp8_rows(oracle.decode(self.pool[rows], "bf16").astype(np.float32))


class MxKeysOfF32Pool:
    """The oracle's MXFP8 quantization of an fp32 key pool, done when indexed (the CPU baseline
    reads only the visible rows of each query): part(0) gives the codes, part(1) the E8M0
    bytes; the two reads of one row set share one quantization."""

    def __init__(self, f32_pool):
        self.pool = f32_pool
        self._last = (None, None)

    def _get(self, rows):
        key = hashlib.sha1(np.ascontiguousarray(rows).tobytes()).digest()
        if self._last[0] != key:
            import oracle
            self._last = (key, oracle.quantize_mxfp8(self.pool[rows]))
        return self._last[1]

    def part(self, i):
        outer = self

        class _Part:
            def __getitem__(self, rows):
                return outer._get(rows)[i]
        return _Part()


def sfa_flops(spec, V):
    return sum(2 * spec.sfa_heads * min(spec.top_k, int(v)) * (spec.d_qk + spec.d_v) for v in V)


def indexer_flops(spec, V):
    return sum(2 * spec.idx_heads * spec.idx_dim * int(v) for v in V)


def source_digest():
    """Digest of the kernel sources' code: comments, blank space and the phase-stamp statements
    (empty in libdsa.so) are dropped first, so that neither detaches the committed counter
    figures from the code they were taken on."""
    h = hashlib.sha256()
    for f in ("indexer.hip", "sfa.hip", "dsa_common.hpp", "dsa_internal.hpp"):
        with open(os.path.join(ROOT, "sparse_indexed_attention_amd", "csrc", f)) as fh:
            src = fh.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        # phase-stamp statements compile to nothing outside the measurement build, and its
        # helpers (the DSA_TIMELINE branch) are not compiled at all
        src = re.sub(r"#ifdef DSA_TIMELINE\b.*?#else\b", " ", src, flags=re.S)
        src = re.sub(r"\btl_(stamp|put|clock)\([^;]*\);", " ", src)
        src = re.sub(r"\btc\.(mark|waited|computed|issued|put)\([^;]*\);", " ", src)
        src = re.sub(r"\bTlCycles tc;", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def counter_traffic(call="indexer"):
    """HBM bytes per launch of one call ("indexer" or "sparse_attn", the latter summing its
    kernels) from the committed rocprofv3 counter summary, if it was taken on the current
    kernel sources; else None."""
    try:
        with open(PROFILE_COUNTERS) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None, None
    if c.get("source_digest") != source_digest() or c.get("workload") is None:
        return None, c.get("workload")
    e = c.get("calls", {}).get(call)
    return (e.get("hbm_bytes_per_launch") if e else None), c.get("workload")


def cpu_baseline(inp, budget_s=12.0):
    """The oracle (NumPy float64, never tuned) on whole queries of the same workload until
    about budget_s of CPU time has passed; queries/s."""
    import oracle
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    threads = cores
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        if info:
            threads = max(int(i.get("num_threads", 1)) for i in info)
    except Exception:
        pass
    T = inp.spec.num_queries
    done = 0
    t0 = time.perf_counter()
    while True:
        t = done % T
        r = oracle.indexer_topk_query(inp, t)
        oracle.sfa_query(inp, t, r.idx)
        done += 1
        if time.perf_counter() - t0 >= budget_s and done >= 1:
            break
    el = time.perf_counter() - t0
    return {"value": done / el, "unit": "queries/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} whole queries (indexer + Top-K + SFA) of the same workload"
                      + (" (each including the oracle's MXFP8 quantization of its visible keys)"
                         if inp.spec.k_dtype == "mxfp8" else "") + ", "
                      f"{el:.1f} s wall, NumPy float64 with {threads} BLAS threads on "
                      f"{cores} available cores"}


def shard_bench(args, dsa, torch, spec, inp, base, lay):
    """The chunk's queries cut into --shards shards (zigzag head-tail pairs from
    dsa_zigzag_ranges, or contiguous ranges); each shard's step (indexer + SFA over just its
    queries) is timed on its own with HIP events, as the share one device of a context-parallel
    group would run.  value = all queries / the sum of the shard times (this one GPU running
    every shard); the per-shard times and their max/min show the balance."""
    G, T, K = args.shards, spec.num_queries, spec.top_k
    shards = []
    for g in range(G):
        if args.layout == "zigzag":
            (b0, e0), (b1, e1) = dsa.zigzag_ranges(T, G, g)
            rows = np.concatenate([np.arange(b0, e0), np.arange(b1, e1)])
        else:
            rows = np.arange(g * T // G, (g + 1) * T // G)
        V = np.asarray(inp.q_visible)[rows]
        o = torch.from_numpy(rows).cuda()
        sub = {f: getattr(base, f)[o].contiguous() for f in ("q_idx", "w", "q_seq", "q_visible", "q_sfa")}
        n = len(rows)
        shards.append(dict(rows=rows, V=V, sub=sub, n=n,
                           ws_i=dsa.zeroed_workspace(dsa.indexer_workspace_bytes(n, int(V.max()), K), "cuda"),
                           ws_s=dsa.zeroed_workspace(dsa.sfa_workspace_bytes(n, spec.sfa_heads, K, spec.d_v), "cuda"),
                           idx=torch.empty((n, K), dtype=torch.int32, device="cuda"),
                           out=torch.empty((n, spec.sfa_heads, spec.d_v), dtype=base.q_sfa.dtype, device="cuda")))

    def run(s, ev=None):
        u = s["sub"]
        if ev:
            ev[0].record()
        dsa.indexer_topk(u["q_idx"], u["w"], base.k_pool, base.k_scale, lay, u["q_seq"], u["q_visible"],
                         int(s["V"].max()), K, out_idx=s["idx"], want_score=False, workspace=s["ws_i"],
                         total_visible=int(s["V"].sum()))
        if ev:
            ev[1].record()
        dsa.sparse_attn(u["q_sfa"], base.kv_pool, s["idx"], lay, u["q_seq"], spec.softmax_scale, spec.d_v,
                        out=s["out"], want_lse=False, workspace=s["ws_s"])
        if ev:
            ev[2].record()

    steps = max(1, args.steps)
    idx_ms, step_ms = [], []
    for s in shards:
        for _ in range(args.warmup):
            run(s)
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        for e in evs:
            run(s, e)
        torch.cuda.synchronize()
        idx_ms.append(float(np.mean([e[0].elapsed_time(e[1]) for e in evs])))
        step_ms.append(float(np.mean([e[0].elapsed_time(e[2]) for e in evs])))
    total_ms = sum(step_ms)
    V_all = [int(v) for v in inp.q_visible]
    idx_tflops = indexer_flops(spec, V_all) / (sum(idx_ms) * 1e-3) / 1e12
    print(f"bench: {G} {args.layout} shards, step ms per shard {[round(x, 3) for x in step_ms]}, "
          f"max/min {max(step_ms) / min(step_ms):.3f}", file=sys.stderr, flush=True)
    line = {
        "metric": METRIC, "value": T / (total_ms * 1e-3), "unit": "queries/s", "n_gpus": 1,
        "steps": steps, "warmup": args.warmup, "ms_per_step": total_ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": spec.name, "queries_per_step": T, "top_k": K,
                   "shards": G, "layout": args.layout,
                   "shard_queries": [s["n"] for s in shards],
                   "shard_causal_positions": [int(s["V"].sum()) for s in shards],
                   "shard_step_ms": step_ms, "shard_indexer_ms": idx_ms,
                   "shard_max_over_min": max(step_ms) / min(step_ms)},
        "roofline": {"bound": "mfma", "kernel": "indexer_topk_kernel", "achieved": idx_tflops,
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": idx_tflops / MFMA_BF16_PEAK_TFLOPS, "traffic": None},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def prolog_bench(args, dsa, torch, spec):
    """dsa_indexer_prolog for the workload's T new tokens (hidden width --prolog-dx, the
    indexer's H x D, keys stored in the workload's key format into a T-row pool), timed with
    HIP events around each call.  Decode is bound by reading the weight matrix (d_x x
    (H D + D + H) bf16); a prefill chunk by the GEMM's MFMA rate."""
    from synth import make_prolog_inputs
    T, H, D, dx = spec.num_queries, spec.idx_heads, spec.idx_dim, args.prolog_dx
    N = H * D + D + H
    pi = make_prolog_inputs(T, dx, H, D, seed=args.seed or 1)
    x = torch.from_numpy(pi.x.view(np.int16)).cuda().view(torch.bfloat16)
    W = torch.from_numpy(pi.w_proj.view(np.int16)).cuda().view(torch.bfloat16)
    g = torch.from_numpy(pi.gain).cuda()
    slot = torch.arange(T, dtype=torch.int64, device="cuda")
    fmt = spec.k_dtype
    if fmt == "fp8":
        pool = torch.zeros((T, D), dtype=torch.uint8, device="cuda")
        ks = torch.zeros((T,), dtype=torch.float32, device="cuda")
        key_bytes = D + 4
    else:
        pool = torch.zeros((T, D), dtype=torch.bfloat16, device="cuda")
        ks, key_bytes = None, 2 * D
    ws = torch.empty(dsa.prolog_workspace_bytes(T, H, D), dtype=torch.uint8, device="cuda")
    q = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
    w = torch.empty((T, H), dtype=torch.float32, device="cuda")
    run = lambda: dsa.indexer_prolog(x, W, g, pi.eps, H, D, slot=slot, k_pool=pool, k_scale=ks,
                                     q_out=q, w_out=w, workspace=ws)
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    steps = max(1, args.steps)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    t0 = time.perf_counter()
    for e in evs:
        e[0].record()
        run()
        e[1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    byts = dx * N * 2 + T * dx * 2 + T * (H * D * 2 + H * 4 + key_bytes) + D * 4
    flops = 2.0 * T * dx * N
    gbs, tfl = byts / (ms * 1e-3) / 1e9, flops / (ms * 1e-3) / 1e12
    # a few tokens reuse no weight: the weight read bounds it; thousands of tokens: the MFMA rate
    hbm = byts / (HBM_PEAK_GBS * 1e9) >= flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    roof = ({"bound": "hbm", "kernel": "indexer prolog (GEMM + epilogue)", "achieved": gbs,
             "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS, "traffic": None}
            if hbm else
            {"bound": "mfma", "kernel": "indexer prolog (GEMM + epilogue)", "achieved": tfl,
             "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": tfl / MFMA_BF16_PEAK_TFLOPS,
             "traffic": None})
    print(f"bench: prolog T={T} d_x={dx} H={H} D={D} keys {fmt}: {ms * 1e3:.1f} us per call, "
          f"{gbs:.0f} GB/s, {tfl:.1f} TFLOP/s", file=sys.stderr, flush=True)
    line = {
        "metric": "indexer prolog tokens/sec (projections + key RMSNorm + key store)",
        "value": T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": spec.name + "_prolog", "tokens": T, "d_x": dx, "heads": H,
                   "head_dim": D, "key_format": fmt, "algorithmic_bytes": byts, "flops": flops,
                   "wall_ms_per_call": wall * 1e3 / steps},
        "roofline": roof, "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def record_timeline(args, dsa, torch, step, spec, V):
    """Phase stamps (include/dsa_timeline.h) of --steps steps: for each, three steps run back to
    back, the stamp buffer is cleared on the stream, and one more step is recorded.  Written to
    args.timeline as JSON: per recorded step and kernel, the stamps of every workgroup that
    started, in microseconds from that step's first indexer start (null: slot not reached);
    the shader-clock counts and readings (slots 8-12, 19), item words (slot 14) and merge flags (slot 15) are kept as
    integers."""
    words = dsa.timeline_bytes() // 8
    buf = torch.zeros(words, dtype=torch.int64, device="cuda")
    dsa.timeline_register(buf)
    kernels = 3
    slots = words // (kernels * 4096)
    steps_out = []
    i = 1000
    for _ in range(max(1, args.steps)):
        for _ in range(3):
            step(i)
            i += 1
        buf.zero_()
        step(i)
        i += 1
        torch.cuda.synchronize()
        a = buf.view(kernels, -1, slots).cpu().numpy()
        starts = a[:, :, 0][a[:, :, 0] > 0]
        if starts.size == 0:
            raise SystemExit("bench: no phase stamps recorded (is DSA_LIB_PATH the timeline build?)")
        first_idx = a[0, :, 0][a[0, :, 0] > 0]
        t0 = int(first_idx.min() if first_idx.size else starts.min())
        rec = {}
        for k, name in enumerate(("indexer", "attention", "combine")):
            wgs = {}
            for wg in np.nonzero(a[k, :, 0])[0]:
                row = a[k, wg]
                # slots 8-12 and 19: shader-clock cycle counts and readings, 14-15: item
                # word and merge flag, kept as integers; the others are stamps
                wgs[int(wg)] = [int(row[s_]) if (8 <= s_ <= 12 or s_ in (14, 15, 19)) else
                                None if row[s_] == 0 else round((int(row[s_]) - t0) * 0.01, 2)
                                for s_ in range(slots)]
            rec[name] = wgs
        steps_out.append(rec)
    dsa.timeline_register(None)
    with open(args.timeline, "w") as f:
        json.dump({"workload": spec.name, "queries": spec.num_queries, "visible": V,
                   "clock": "s_memrealtime, 100 MHz", "steps": steps_out}, f)
    print(f"bench: {len(steps_out)} recorded steps written to {args.timeline}", file=sys.stderr,
          flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=4, help="workload number (1-6)")
    ap.add_argument("--copies", type=int, default=0, help="rotating input copies (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--sfa-kv", choices=("bf16", "fp8"), default="bf16",
                    help="latent cache storage read by SFA")
    ap.add_argument("--idx-keys", choices=("default", "mxfp8"), default="default",
                    help="index key storage (default: the workload's)")
    ap.add_argument("--shards", type=int, default=0,
                    help="time the workload cut into this many shards of queries, one after the "
                         "other (each one device's share at its real shape)")
    ap.add_argument("--layout", choices=("zigzag", "contiguous"), default="zigzag",
                    help="how --shards cuts the chunk of queries")
    ap.add_argument("--ctx", type=int, default=0,
                    help="decode workloads: give every sequence this many tokens (e.g. 131072 for "
                         "the 128K end of workload 4's range); the workload is renamed *_ctxN")
    ap.add_argument("--order", choices=("natural", "zigzag"), default="natural",
                    help="query order of the unsharded launch: zigzag pairs the 4-query tiles "
                         "head and tail (0, B-1, 1, B-2, ...), the workgroup-level pairing of short "
                         "and long causal histories; it changes only the order (and so the timing)")
    ap.add_argument("--prolog", action="store_true",
                    help="time the indexer prolog (projections, key RMSNorm, query quantization, "
                         "key store) for the workload's new tokens instead of the step")
    ap.add_argument("--prolog-dx", type=int, default=7168, help="hidden width for --prolog")
    ap.add_argument("--timeline", default="", metavar="PATH",
                    help="with the measurement build (DSA_LIB_PATH=.../libdsa_timeline.so): record "
                         "the kernels' per-workgroup phase stamps of --steps steps (each after three "
                         "untimed ones) into PATH as JSON instead of timing")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB three times (the "
                         "reference kernel for scaling the HBM byte counters) and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (a causal chunk "
              "can be sharded across devices with dsa_zigzag_ranges; --shards times each "
              "shard's share on this GPU).", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "copies": 3}), flush=True)
        return
    import sparse_indexed_attention_amd as dsa
    from synth import make_inputs, workload
    from synth.device import to_device

    dsa.load()
    torch.cuda.set_device(0)
    spec = workload(args.config)
    if args.ctx:
        if spec.name.startswith("prefill"):
            raise SystemExit("bench: --ctx applies to the decode workloads")
        from synth import scaled_spec
        spec = scaled_spec(spec, seq_lens=[args.ctx] * spec.num_seqs,
                           name=f"{spec.name}_ctx{args.ctx}")
    if args.prolog:
        prolog_bench(args, dsa, torch, spec)
        return
    seed = args.seed or args.config
    print(f"bench: generating {spec.name} (seed {seed})", file=sys.stderr, flush=True)
    mx_keys = args.idx_keys == "mxfp8"
    if mx_keys:
        spec = dataclasses.replace(spec, k_dtype="f32")
    inp = make_inputs(spec, seed=seed)
    if args.sfa_kv == "fp8":
        spec = dataclasses.replace(spec, kv_dtype="fp8", name=spec.name + "_fp8kv")
        inp = dataclasses.replace(inp, spec=spec, kv_pool=Fp8RowsOfBf16Pool(inp.kv_pool))
    V = [int(v) for v in inp.q_visible]
    total_visible = sum(V)       # known to the host, as in a serving scheduler
    T = spec.num_queries

    step_bytes_idx = indexer_bytes(dataclasses.replace(spec, k_dtype="mxfp8") if mx_keys else spec, V)
    step_bytes_sfa = sfa_bytes(spec, V)
    per_copy = step_bytes_idx + step_bytes_sfa
    copies = args.copies or max(3, min(12, math.ceil(1.0e9 / per_copy) + 1))
    if spec.name.startswith("prefill"):
        copies = args.copies or 1
    if args.sfa_kv == "fp8":
        bf16_pool = inp.kv_pool.pool
        inp.kv_pool = bf16_pool
        base = to_device(inp, "cuda")
        n = base.kv_pool.shape[0]
        pool8 = torch.zeros((n, KV_FP8_ROW_BYTES), dtype=torch.uint8, device="cuda")
        dsa.store_kv(base.kv_pool, torch.arange(n, dtype=torch.int64, device="cuda"), pool8)
        torch.cuda.synchronize()
        base.kv_pool = pool8
        inp.kv_pool = Fp8RowsOfBf16Pool(bf16_pool)
    else:
        base = to_device(inp, "cuda")
    if mx_keys:
        # the product's cache writer quantizes the fp32 keys on the GPU; the CPU baseline gets
        # the oracle's quantization of the same keys
        n, D = base.k_pool.shape
        kp = torch.zeros((n, D), dtype=torch.uint8, device="cuda")
        ks = torch.zeros((n, D // 32), dtype=torch.uint8, device="cuda")
        dsa.store_index_keys(base.k_pool, torch.arange(n, dtype=torch.int64, device="cuda"), kp, ks)
        torch.cuda.synchronize()
        base.k_pool, base.k_scale = kp, ks
        spec = dataclasses.replace(spec, k_dtype="mxfp8", name=spec.name + "_mxkeys")
        mxq = MxKeysOfF32Pool(inp.k_pool)
        inp = dataclasses.replace(inp, spec=spec, k_pool=mxq.part(0), k_scale=mxq.part(1))
    devs = [base]
    for _ in range(copies - 1):
        c = copy.copy(base)
        for f in ("q_idx", "w", "k_pool", "k_scale", "q_sfa", "kv_pool", "block_table", "q_seq",
                  "q_visible"):
            v = getattr(base, f)
            setattr(c, f, None if v is None else v.clone())
        devs.append(c)
    layouts = [dsa.make_layout(d.block_table, d.block_size, pool_rows=d.pool_rows)
               if d.block_table is not None else
               dsa.make_layout(None, 0, seq_stride=d.seq_stride, num_seqs=spec.num_seqs,
                               pool_rows=d.pool_rows) for d in devs]
    K = spec.top_k
    if args.shards:
        shard_bench(args, dsa, torch, spec, inp, base, layouts[0])
        return
    if args.order == "zigzag":
        # tiles of 4 consecutive queries (one multi-query indexer workgroup each) in head-tail
        # order; every copy of the inputs is permuted the same way
        nb = (T + 3) // 4
        blocks = [b for i in range((nb + 1) // 2) for b in ((i, nb - 1 - i) if i != nb - 1 - i else (i,))]
        perm = torch.tensor([q for b in blocks for q in range(4 * b, min(T, 4 * b + 4))],
                            dtype=torch.int64, device="cuda")
        for d in devs:
            for f in ("q_idx", "w", "q_sfa", "q_seq", "q_visible"):
                setattr(d, f, getattr(d, f).index_select(0, perm).contiguous())
        args.no_cpu_baseline = True
    ws_i = dsa.zeroed_workspace(dsa.indexer_workspace_bytes(T, base.max_visible, K), "cuda")
    ws_s = dsa.zeroed_workspace(dsa.sfa_workspace_bytes(T, spec.sfa_heads, K, spec.d_v), "cuda")
    outs = []
    for d in devs:
        # valid index lists from the start (position 0 repeated), so that the attention call can
        # be timed on every copy before the indexer has written it
        idx = torch.zeros((T, K), dtype=torch.int32, device="cuda")
        o = torch.empty((T, spec.sfa_heads, spec.d_v), dtype=d.q_sfa.dtype, device="cuda")
        outs.append((idx, o))

    def call_idx(i):
        d, lay = devs[i % copies], layouts[i % copies]
        dsa.indexer_topk(d.q_idx, d.w, d.k_pool, d.k_scale, lay, d.q_seq, d.q_visible,
                         d.max_visible, K, out_idx=outs[i % copies][0], want_score=False,
                         workspace=ws_i, total_visible=total_visible)

    def call_sfa(i):
        d, lay = devs[i % copies], layouts[i % copies]
        idx, o = outs[i % copies]
        dsa.sparse_attn(d.q_sfa, d.kv_pool, idx, lay, d.q_seq, spec.softmax_scale, spec.d_v,
                        out=o, want_lse=False, workspace=ws_s)

    def step(i):
        call_idx(i)
        call_sfa(i)

    print(f"bench: {copies} rotating copies, warmup {args.warmup}", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    if args.timeline:
        record_timeline(args, dsa, torch, step, spec, V)
        return

    # The timed region: exactly --steps steps between two synchronizations, nothing else.
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    t_host = time.perf_counter() - t0
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = wall * 1e3 / args.steps
    qps = T * args.steps / wall

    # Per-call times, after the timed region: each call alone, launched back to back over the
    # rotating copies.  A GPU sleep queued first keeps the device busy while the host enqueues
    # every launch, so the events see a full queue (never an idle GPU waiting for the host);
    # one event between batches of BATCH calls gives BATCHES samples of the mean call time.
    BATCHES, BATCH = (60, 8) if step_ms < 1.0 else (12, 1)

    def per_call_us(fn):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(BATCHES + 1)]
        torch.cuda.synchronize()
        try:
            torch.cuda._sleep(int(2.4e9 * 0.05))   # ~50 ms at 2.4 GHz, longer than the enqueueing
        except (AttributeError, RuntimeError):
            print("bench: no GPU sleep available; per-call times may include host gaps",
                  file=sys.stderr, flush=True)
        evs[0].record()
        n = 0
        for b in range(BATCHES):
            for _ in range(BATCH):
                fn(n)
                n += 1
            evs[b + 1].record()
        torch.cuda.synchronize()
        return np.array([evs[b].elapsed_time(evs[b + 1]) * 1e3 / BATCH for b in range(BATCHES)])

    idx_us = per_call_us(call_idx)
    sfa_us = per_call_us(call_sfa)

    def stats(us):
        return {"mean": float(us.mean()), "median": float(np.median(us)), "min": float(us.min()),
                "p10": float(np.percentile(us, 10)), "p90": float(np.percentile(us, 90)),
                "samples": int(us.size), "calls_per_sample": BATCH}

    idx_mean = float(idx_us.mean()) * 1e-3          # ms
    sfa_mean = float(sfa_us.mean()) * 1e-3
    # the two calls run back to back in a step, so their separate times cannot exceed it
    # (medians, robust to a slow sample; 5% allowed for run-to-run noise between the two
    # measurements)
    consistent = (float(np.median(idx_us)) + float(np.median(sfa_us))) * 1e-3 <= step_ms * 1.05
    achieved = step_bytes_idx / (idx_mean * 1e-3) / 1e9
    # counter-measured bytes only for the workload the committed counters were taken on
    traffic, prof_wl = counter_traffic("indexer")
    sfa_traffic, _ = counter_traffic("sparse_attn")
    if prof_wl != spec.name:
        traffic = sfa_traffic = None
    print(f"bench: step {step_ms * 1e3:.1f} us (host enqueue {t_host * 1e6 / args.steps:.1f} us); "
          f"indexer {idx_mean * 1e3:.1f} us (median {np.median(idx_us):.1f}, p10 "
          f"{np.percentile(idx_us, 10):.1f}, p90 {np.percentile(idx_us, 90):.1f}), "
          f"{achieved:.0f} GB/s; SFA {sfa_mean * 1e3:.1f} us, "
          f"{step_bytes_sfa / (sfa_mean * 1e-3) / 1e9:.0f} GB/s, "
          f"{sfa_flops(spec, V) / (sfa_mean * 1e-3) / 1e12:.1f} TFLOP/s; whole step "
          f"{(step_bytes_idx + step_bytes_sfa) / (step_ms * 1e-3) / 1e9:.0f} GB/s",
          file=sys.stderr, flush=True)
    if not consistent:
        print(f"bench: ERROR: indexer {np.median(idx_us):.1f} us + SFA {np.median(sfa_us):.1f} us (medians) exceed "
              f"the step's {step_ms * 1e3:.1f} us", file=sys.stderr, flush=True)
        sys.exit(3)

    cpu = None
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle", file=sys.stderr, flush=True)
        cpu = cpu_baseline(inp, args.cpu_budget)

    # The indexer is the dominant kernel.  Decode streams every key once (HBM-bound); in chunked
    # prefill thousands of queries share one cached context, so the key bytes are reused from
    # the caches and the bound is the MFMA rate on its 2*H*D flops per visible position.
    prefill = spec.name.startswith("prefill")
    sfa_tflops = sfa_flops(spec, V) / (sfa_mean * 1e-3) / 1e12
    if prefill:
        idx_tflops = indexer_flops(spec, V) / (idx_mean * 1e-3) / 1e12
        roofline = {"bound": "mfma", "kernel": "indexer_topk_kernel", "achieved": idx_tflops,
                    "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": idx_tflops / MFMA_BF16_PEAK_TFLOPS, "traffic": None}
        sfa_roof = {"bound": "mfma", "kernel": "sfa (attention + fixup)", "achieved": sfa_tflops,
                    "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": sfa_tflops / MFMA_BF16_PEAK_TFLOPS}
    else:
        roofline = {"bound": "hbm", "kernel": "indexer_topk_kernel", "achieved": achieved,
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                    "traffic": traffic}
        sfa_gbs = step_bytes_sfa / (sfa_mean * 1e-3) / 1e9
        sfa_roof = {"bound": "hbm", "kernel": "sfa (attention + combine)", "achieved": sfa_gbs,
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": sfa_gbs / HBM_PEAK_GBS,
                    "traffic": sfa_traffic, "tflops": sfa_tflops}
    step_cfg = {}
    if not prefill:
        # a decode step streams its bytes from HBM; a prefill chunk reuses its cached context
        # from the caches, so there the byte count is not an HBM figure
        step_cfg = {"step_algorithmic_bytes": step_bytes_idx + step_bytes_sfa,
                    "step_hbm_frac": (step_bytes_idx + step_bytes_sfa) / (step_ms * 1e-3) / 1e9
                    / HBM_PEAK_GBS}
    line = {
        "metric": METRIC,
        "value": qps,
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": spec.name,
            "query_order": args.order,
            "queries_per_step": T,
            "context": {"min": min(V), "max": max(V), "mean": float(np.mean(V))},
            "top_k": K,
            "indexer": f"{spec.idx_heads}x{spec.idx_dim} q {spec.q_dtype} keys {spec.k_dtype}",
            "sfa": f"{spec.sfa_heads} heads {spec.d_qk}/{spec.d_v} {spec.kv_dtype}",
            "block_size": spec.block_size,
            "rotating_copies": copies,
            **step_cfg,
            "indexer_us": stats(idx_us),
            "sfa_us": stats(sfa_us),
            "sfa_roofline": sfa_roof,
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
