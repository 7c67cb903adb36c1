#!/usr/bin/env python3
"""Benchmark of the few-row quantized GEMV on one MI355X.

Workload (default): the square projection K = N = 4096, 4-bit affine codes,
group size 64, activation rows M in {1, 2, 3, 4, 5, 8}.  One step = one
verify call per M (dispatcher's choice of path), each on the next weight copy
of a rotating pool larger than every cache (>= 1 GiB, well above the 256 MB
MALL), so every call streams its weights from HBM.

Timing: the K timed steps are captured into one HIP graph (a dependent chain
of launches on one stream, no host in the loop) and replayed between two
events after W warm-up steps.  Per-cell chains (one graph of L launches for
each M and each forced path, walked in interleaved rounds, median over the
rounds) give time(M)/time(1) for the dispatcher's choice and for each path,
and the average launch duration of each kernel.

Prints ONE JSON line (rank 0).  --gpus N with N > 1 exits with a message:
the library runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from few_row_quantized_amd import accounting, synth  # noqa: E402

METRIC = "effective weight GB/s (% of HBM peak) and time(M)/time(1) at M=1..16"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK = 2.5e15  # dense bf16 MFMA flop/s of one MI355X


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="square_k4096_n4096_4b_g64")
    ap.add_argument("--m-values", default=None, help="comma list; default: the workload's")
    ap.add_argument("--pool-mib", type=int, default=1024)
    ap.add_argument("--chain", type=int, default=400, help="launches per per-cell chain")
    ap.add_argument("--rounds", type=int, default=5, help="interleaved rounds over the cells")
    ap.add_argument("--path", default="auto", choices=["auto", "dot", "mfma"])
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU oracle budget")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--hot", action="store_true", help="reuse one weight copy (cache-resident)")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the streaming-read ceiling")
    ap.add_argument("--no-residual", action="store_true",
                    help="skip the fused residual sum (MUL_MAT + ADD) comparison")
    ap.add_argument("--no-moe", action="store_true",
                    help="skip the gathered (MoE) verify measurement")
    return ap.parse_args()


class Pool:
    """P device copies of (codes, scales, biases) with identical contents."""

    def __init__(self, p, copies):
        import numpy as np
        import torch
        self.P = copies
        c = torch.from_numpy(p.codes).cuda()
        fp = p.shape.fmt is not None  # block-scaled FP: scale bytes, no biases
        s = torch.from_numpy(p.scales if fp else p.scales.view(np.int16)).cuda()
        b = torch.from_numpy(p.biases.view(np.int16)).cuda()
        self.codes = torch.empty((copies,) + tuple(c.shape), dtype=c.dtype, device="cuda")
        self.scales = torch.empty((copies,) + tuple(s.shape), dtype=s.dtype, device="cuda")
        self.biases = torch.empty((copies,) + tuple(b.shape), dtype=b.dtype, device="cuda")
        for i in range(copies):
            self.codes[i].copy_(c)
            self.scales[i].copy_(s)
            self.biases[i].copy_(b)
        torch.cuda.synchronize()


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the library runs on one GPU; --gpus must be 1",
                          "n_gpus_requested": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch
    from few_row_quantized_amd import qgemv as q

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    q.lib()  # fail loudly if the library is missing

    s = synth.WORKLOADS[args.workload]
    ms = [int(v) for v in args.m_values.split(",")] if args.m_values else list(s.m_values)
    p = synth.make_problem(s, m_max=max(ms))
    fp = s.fmt is not None
    W = (accounting.fp_weight_bytes(s.N, s.K, s.bits, s.group_size) if fp else
         accounting.weight_bytes(s.N, s.K, s.bits, s.group_size))
    copies = 1 if args.hot else max(2, math.ceil(args.pool_mib * 2 ** 20 / W))
    log(f"[bench] {s.name}: W={W} B, pool of {copies} copies ({copies * W / 2**20:.0f} MiB), M={ms}")
    pool = Pool(p, copies)
    x = torch.from_numpy(p.x.view(np.int16)).cuda()
    ys = {M: torch.empty((M, s.N), dtype=torch.float32, device="cuda") for M in ms}
    def select(M):
        return q.qgemv_select_fp(M, s.N, s.K, s.fmt) if fp else q.qgemv_select(M, s.N, s.K, s.bits,
                                                                               s.group_size)

    def supported(path, M):
        return (q.qgemv_path_supported_fp(path, M, s.N, s.K, s.fmt) if fp else
                q.qgemv_path_supported(path, M, s.N, s.K, s.bits, s.group_size))

    paths = {M: (args.path if args.path != "auto" else {q.PATH_DOT: "dot", q.PATH_MFMA: "mfma"}[select(M)])
             for M in ms}

    counter = [0]

    def call(path, i, M, y, residual=None):
        if fp:
            q.qgemv_run_path_fp(path, pool.codes[i], pool.scales[i], x, residual, y, M, s.N, s.K, s.fmt)
        elif residual is not None:
            q.qgemv_run_path_add(path, pool.codes[i], pool.scales[i], pool.biases[i], x, residual, y,
                                 M, s.N, s.K, s.bits, s.group_size)
        else:
            q.qgemv_run_path(path, pool.codes[i], pool.scales[i], pool.biases[i], x, y, M, s.N, s.K,
                             s.bits, s.group_size)

    def launch(M, path=args.path):
        i = counter[0] % copies
        counter[0] += 1
        call(path, i, M, ys[M])

    def alg_bytes(M):
        return (accounting.fp_algorithmic_bytes(M, s.N, s.K, s.bits, s.group_size) if fp else
                accounting.algorithmic_bytes(M, s.N, s.K, s.bits, s.group_size))

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        return g

    def time_graph(g, reps=1):
        # the kernels run on torch's current stream, which is where these events are recorded
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3  # seconds

    # eager warm-up (first launches load code objects)
    for M in ms:
        launch(M)
    torch.cuda.synchronize()

    # main measurement: K steps in one graph, W warm-up steps in another
    warm_g = capture(lambda: [launch(M) for _ in range(max(1, args.warmup)) for M in ms])
    main_g = capture(lambda: [launch(M) for _ in range(args.steps) for M in ms])
    log("[bench] graphs captured; warm-up")
    time_graph(warm_g)
    log(f"[bench] timing {args.steps} steps")
    t_main = time_graph(main_g)
    ms_per_step = t_main / args.steps * 1e3
    value = (W * len(ms) * args.steps) / t_main / 1e9

    # per-cell chains, one cell per (M, forced path): one graph of `chain`
    # launches each, replayed once to warm up and then once per round, the
    # rounds walking every cell in turn (interleaved), median over rounds
    forced = ["dot", "mfma"] if args.path == "auto" else [args.path]
    cells = [(M, pth) for M in ms for pth in forced if supported(pth, M)]
    graphs = {c: capture(lambda c=c: [launch(c[0], c[1]) for _ in range(args.chain)]) for c in cells}
    for c in cells:
        time_graph(graphs[c])
    samples = {c: [] for c in cells}
    for _ in range(args.rounds):
        for c in cells:
            samples[c].append(time_graph(graphs[c]) / args.chain)
    t_cell = {c: statistics.median(v) for c, v in samples.items()}
    del graphs

    ceiling = None if args.no_ceiling else measure_ceiling(W, copies, args.chain, capture, time_graph)
    residual = None
    if not args.no_residual:
        residual = measure_residual_sum(s, p, ms, paths, call, copies, args, capture, time_graph)
    moe = None
    if not args.no_moe:
        del pool
        torch.cuda.empty_cache()
        moe = measure_moe(args, capture, time_graph)

    def cell_json(M, pth, t, t1):
        alg = alg_bytes(M)
        d = {"path": pth, "us": round(t * 1e6, 4),
             "us_min_max_over_rounds": [round(min(samples[(M, pth)]) * 1e6, 4),
                                        round(max(samples[(M, pth)]) * 1e6, 4)],
             "weight_GBps": round(W / t / 1e9, 1),
             "pct_hbm_peak": round(100 * W / t / 1e9 / HBM_PEAK_GBS, 2),
             "alg_GBps": round(alg / t / 1e9, 1),
             "t_over_t1": round(t / t1, 4) if t1 else None,
             "mfma_util_useful": round(accounting.useful_flops(M, s.N, s.K) / t / MFMA_BF16_PEAK, 6),
             "mfma_util_issued": round(2 * 16 * s.N * s.K / t / MFMA_BF16_PEAK, 6)
             if pth == "mfma" else 0.0}
        if ceiling:
            d["pct_stream_probe"] = round(100 * ceiling["stream_probe_us"] / (t * 1e6), 2)
        return d

    # the dispatcher's choice per M is one of the forced cells (the same launch)
    per_m = {M: t_cell[(M, paths[M])] for M in ms}
    for M in ms:
        log(f"[bench] M={M:2d} path={paths[M]:4s} {per_m[M] * 1e6:8.3f} us/launch  "
            f"{W / per_m[M] / 1e9:8.1f} GB/s")
    t1 = per_m.get(1, per_m[min(ms)])
    per_m_json = {str(M): cell_json(M, paths[M], per_m[M], t1) for M in ms}
    forced_json = {}
    for pth in forced:
        mp = [M for M in ms if (M, pth) in t_cell]
        if mp:
            t1p = t_cell[(min(mp), pth)] if min(mp) == min(ms) else None
            forced_json[pth] = {str(M): cell_json(M, pth, t_cell[(M, pth)], t1p) for M in mp}

    # dominant kernel = the (path, M) configuration with the largest time per step
    Mdom = max(ms, key=lambda M: per_m[M])
    alg = alg_bytes(Mdom)
    achieved = alg / per_m[Mdom] / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(s.name, Mdom, paths[Mdom]),
                "kernel": f"{paths[Mdom]} path M={Mdom}",
                "bytes_per_launch": alg, "avg_launch_us": round(per_m[Mdom] * 1e6, 4)}
    # the same figure from the committed rocprofv3 trace's average kernel
    # duration (no launch gaps; the profiler's own overhead included)
    prof = profiled_kernel_us(s.name, Mdom, paths[Mdom])
    if prof:
        a_p = alg / (prof["avg_us"] * 1e-6) / 1e9
        roofline.update({"achieved_rocprof": round(a_p, 1), "frac_rocprof": round(a_p / HBM_PEAK_GBS, 4),
                         "rocprof_avg_us": prof["avg_us"], "rocprof_kernel": prof["kernel"],
                         "rocprof_dispatches": prof["dispatches"], "rocprof_file": prof["file"]})
    if ceiling:
        roofline["frac_of_stream_probe"] = round(ceiling["stream_probe_us"] / (per_m[Mdom] * 1e6), 4)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(p, ms, W, args.cpu_seconds)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": s.name, "K": s.K, "N": s.N, "bits": s.bits,
                   "group_size": s.group_size, "format": s.fmt or "affine", "m_values": ms, "path": args.path,
                   "weight_bytes": W, "pool_copies": copies, "seed": p.seed,
                   "timing": "one HIP graph of K steps; each call on the next pool copy"},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "t8_over_t1": per_m_json.get("8", {}).get("t_over_t1"),
        "per_m": per_m_json,
        "forced_paths": forced_json,
        "schedule": {"cells": [list(c) for c in cells], "rounds": args.rounds, "chain": args.chain},
        "roofline": roofline,
        "ceiling": ceiling,
        "residual_sum": residual,
        "moe_verify": moe,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def measure_residual_sum(s, p, ms, paths, call, copies, args, capture, time_graph):
    """The fused residual sum y = x W^T + r against the plain product and
    against the plain product followed by a separate fp32 add (torch's
    elementwise kernel, i.e. the unfused MUL_MAT then ADD): per M, the
    dispatcher's path, chains of `chain` launches on the rotating pool,
    interleaved rounds, median over rounds."""
    import numpy as np
    import torch
    from few_row_quantized_amd import qgemv as q
    r = torch.from_numpy(synth.make_residual(max(ms), s.N, seed=p.seed)).cuda()
    rs = {M: r[:M].contiguous() for M in ms}
    ys = {M: torch.empty((M, s.N), dtype=torch.float32, device="cuda") for M in ms}
    ts = {M: torch.empty((M, s.N), dtype=torch.float32, device="cuda") for M in ms}
    ctr = [0]

    def one(M, kind):
        i = ctr[0] % copies
        ctr[0] += 1
        if kind == "fused":
            call(paths[M], i, M, ys[M], residual=rs[M])
        else:
            call(paths[M], i, M, ts[M])
            if kind == "separate":
                torch.add(ts[M], rs[M], out=ys[M])

    kinds = ("plain", "fused", "separate")
    cells = [(M, k) for M in ms for k in kinds]
    for c in cells:
        one(*c)
    torch.cuda.synchronize()
    graphs = {c: capture(lambda c=c: [one(*c) for _ in range(args.chain)]) for c in cells}
    for c in cells:
        time_graph(graphs[c])
    samp = {c: [] for c in cells}
    for _ in range(args.rounds):
        for c in cells:
            samp[c].append(time_graph(graphs[c]) / args.chain)
    del graphs
    out = {}
    for M in ms:
        t = {k: statistics.median(samp[(M, k)]) * 1e6 for k in kinds}
        out[str(M)] = {"path": paths[M], "plain_us": round(t["plain"], 4),
                       "fused_us": round(t["fused"], 4), "separate_add_us": round(t["separate"], 4),
                       "saved_us": round(t["separate"] - t["fused"], 4),
                       "fused_over_plain": round(t["fused"] / t["plain"], 4)}
        log(f"[bench] residual sum M={M:2d} plain {t['plain']:.3f} fused {t['fused']:.3f} "
            f"plain+add {t['separate']:.3f} us")
    # the fused result is the plain product plus r rounded once: check it
    for M in ms:
        one(M, "fused")
        one(M, "plain")
    torch.cuda.synchronize()
    exact = all(np.array_equal(ys[M].cpu().numpy(), (ts[M] + rs[M]).cpu().numpy()) for M in ms)
    return {"per_m": out, "bitwise_plain_plus_add": exact,
            "timing": "graph chains per (M, variant), interleaved rounds, median; "
                      "separate = plain call then torch.add(y, r)"}


def measure_moe(args, capture, time_graph, name="moe30b_gateup_e128_k2048_n1536_4b_g64_top8",
                ms=(1, 2, 4, 8, 16)):
    """Gathered (MoE) verify: per M, one qgemv_gather call over the M*topk
    (row, expert) pairs, which reads each expert of the union once, against M
    calls of one row each (the routed experts streamed once per verify row).
    Weights rotate over copies of the expert set larger than the caches;
    chains of launches, interleaved rounds, median."""
    import numpy as np
    import torch
    from few_row_quantized_amd import qgemv as q
    sh = synth.MOE_WORKLOADS[name]
    p = synth.make_moe_problem(sh, m_max=max(ms))
    expert_bytes = accounting.weight_bytes(sh.N, sh.K, sh.bits, sh.group_size)
    total = expert_bytes * sh.E
    copies = max(2, math.ceil(args.pool_mib * 2 ** 20 / total))
    codes = torch.from_numpy(p.codes).cuda()
    sc = torch.from_numpy(p.scales.view(np.int16)).cuda()
    bi = torch.from_numpy(p.biases.view(np.int16)).cuda()
    pool = [(codes, sc, bi)] + [(codes.clone(), sc.clone(), bi.clone()) for _ in range(copies - 1)]
    x = torch.from_numpy(p.x.view(np.int16)).cuda()
    ys = torch.empty((sh.topk * max(ms), sh.N), dtype=torch.float32, device="cuda")
    pairs = {}
    for M in ms:
        xi, ei = p.pairs(M)
        pairs[M] = (torch.from_numpy(xi).cuda(), torch.from_numpy(ei).cuda(), len(set(ei.tolist())))
    rows = {m: (torch.from_numpy(np.zeros(sh.topk, np.int32)).cuda(),
                torch.from_numpy(p.routing[m].astype(np.int32)).cuda()) for m in range(max(ms))}
    ctr = [0]

    def one(M, kind):
        c = pool[ctr[0] % copies]
        ctr[0] += 1
        if kind == "gathered":
            xi, ei, _ = pairs[M]
            q.qgemv_gather(c[0], c[1], c[2], x, xi, ei, ys, len(xi), M, sh.E, sh.N, sh.K, sh.bits,
                           sh.group_size)
        else:
            for m in range(M):
                xi, ei = rows[m]
                q.qgemv_gather(c[0], c[1], c[2], x[m:m + 1], xi, ei, ys[sh.topk * m:], sh.topk, 1,
                               sh.E, sh.N, sh.K, sh.bits, sh.group_size)

    chain = max(20, args.chain // 8)
    cells = [(M, k) for M in ms for k in ("gathered", "per_row")]
    for c in cells:
        one(*c)
    torch.cuda.synchronize()
    graphs = {c: capture(lambda c=c: [one(*c) for _ in range(chain)]) for c in cells}
    for c in cells:
        time_graph(graphs[c])
    samp = {c: [] for c in cells}
    for _ in range(args.rounds):
        for c in cells:
            samp[c].append(time_graph(graphs[c]) / chain)
    del graphs
    out = {}
    t1 = None
    for M in ms:
        tg = statistics.median(samp[(M, "gathered")])
        tr = statistics.median(samp[(M, "per_row")])
        t1 = t1 or tg
        union = pairs[M][2]
        out[str(M)] = {"pairs": M * sh.topk, "union_experts": union, "gathered_us": round(tg * 1e6, 3),
                       "per_row_us": round(tr * 1e6, 3), "speedup": round(tr / tg, 3),
                       "t_over_t1": round(tg / t1, 3),
                       "union_GBps": round(union * expert_bytes / tg / 1e9, 1),
                       "us_per_verify_row": round(tg * 1e6 / M, 3)}
        log(f"[bench] moe M={M:2d} pairs={M * sh.topk:3d} union={union:3d} gathered {tg * 1e6:8.2f} us "
            f"per-row {tr * 1e6:8.2f} us  {union * expert_bytes / tg / 1e9:7.1f} GB/s")
    del pool
    torch.cuda.empty_cache()
    return {"workload": name, "experts": sh.E, "topk": sh.topk, "expert_bytes": expert_bytes,
            "pool_copies": copies, "per_m": out,
            "timing": "graph chains; gathered = one qgemv_gather per verify step; per_row = M calls of "
                      "one row's 8 pairs; interleaved rounds, median"}


def csrc_sha256():
    """sha256 of the kernel sources with comments and blank lines removed: a
    profile stays valid across edits of comments only, and goes stale with
    any change of code."""
    import glob
    import hashlib
    import re
    srcs = sorted(glob.glob(os.path.join(ROOT, "few_row_quantized_amd", "csrc", "*")))
    h = hashlib.sha256()
    for f in srcs:
        text = open(f, encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)  # block comments
        text = re.sub(r"//[^\n]*", "", text)                # line comments
        lines = [ln.rstrip() for ln in text.splitlines() if ln.strip()]
        h.update(os.path.basename(f).encode() + b"\0" + "\n".join(lines).encode() + b"\0")
    return h.hexdigest()


def profiled_kernel_us(workload, M, path):
    """Average duration (us) of the (path, M) cell's GEMV kernel in the
    committed rocprofv3 kernel trace of this workload (start to end of each
    dispatch, the timed chains of a bench run under the profiler), with the
    file it comes from.  None when no such trace exists or when the kernel
    sources changed since it was taken."""
    rel = os.path.join("profiles", f"kernel_trace_{workload}.json")
    path_json = os.path.join(ROOT, rel)
    if not os.path.exists(path_json):
        return None
    rec = json.load(open(path_json))
    cell = rec.get("cells", {}).get(f"{path}/{M}")
    if rec.get("csrc_sha256") != csrc_sha256() or cell is None:
        return None
    return {"avg_us": cell["avg_us"], "dispatches": cell["dispatches"], "kernel": cell["kernel"],
            "file": rel}


def measured_traffic(workload, M, path):
    """HBM bytes per launch (read + write) of the (path, M) cell from the
    committed rocprofv3 FETCH_SIZE / WRITE_SIZE passes for this workload,
    each scaled by the counters' reading of a device copy of known size in
    the same run.  None when no such profile exists or when the kernel
    sources changed since it was taken."""
    fn = os.path.join(ROOT, "profiles", f"counters_{workload}.json")
    if not os.path.exists(fn):
        return None
    rec = json.load(open(fn))
    t = rec.get("cells", {}).get(f"{path}/{M}")
    if rec.get("csrc_sha256") != csrc_sha256() or t is None or t.get("read_bytes") is None:
        return None
    return t["read_bytes"] + t["write_bytes"]


def measure_ceiling(W, copies, chain, capture, time_graph):
    """Pure streaming read of W bytes per launch (qgemv_stream_probe) over the
    same rotating-pool protocol, for each layout and loads-per-thread setting
    of the probe; the ceiling is the fastest.  Also the same probe on a tiny
    buffer (the per-launch floor of a graph chain)."""
    import torch
    from few_row_quantized_amd import qgemv as q
    nbytes = (W + 15) // 16 * 16
    buf = torch.randint(0, 255, (copies, nbytes), dtype=torch.uint8, device="cuda")
    out = torch.empty(q.qgemv_stream_probe_blocks(nbytes), dtype=torch.int32, device="cuda")
    small = 64 * 1024
    sout = torch.empty(q.qgemv_stream_probe_blocks(small), dtype=torch.int32, device="cuda")
    ctr = [0]
    per_cfg = {}
    for layout in (0, 1):
        for u in (1, 2, 4, 8, 16):
            def one(u=u, layout=layout):
                i = ctr[0] % copies
                ctr[0] += 1
                q.qgemv_stream_probe(buf[i], nbytes, out, u, layout)

            one()
            g = capture(lambda: [one() for _ in range(chain)])
            time_graph(g)
            per_cfg[(layout, u)] = time_graph(g, reps=2) / (2 * chain)
    best = min(per_cfg, key=per_cfg.get)
    t = per_cfg[best]
    gs = capture(lambda: [q.qgemv_stream_probe(buf[0], small, sout, 4, 0) for _ in range(chain)])
    time_graph(gs)
    tf = time_graph(gs, reps=2) / (2 * chain)
    names = {0: "grid-stride", 1: "wave-contiguous"}
    log(f"[bench] stream probe {nbytes} B: best {t * 1e6:.3f} us/launch ({names[best[0]]}, {best[1]} "
        f"loads/thread) = {nbytes / t / 1e9:.1f} GB/s; "
        + ", ".join(f"{names[l]}/{u}: {v * 1e6:.3f}" for (l, u), v in per_cfg.items())
        + f"; 64 KiB floor {tf * 1e6:.3f} us")
    del buf
    return {"stream_probe_bytes": nbytes, "stream_probe_us": round(t * 1e6, 4),
            "stream_probe_GBps": round(nbytes / t / 1e9, 1),
            "stream_probe_layout": names[best[0]], "stream_probe_loads_per_thread": best[1],
            "stream_probe_us_by_setting": {f"{names[l]}/{u}": round(v * 1e6, 4)
                                           for (l, u), v in per_cfg.items()},
            "launch_floor_us_64KiB": round(tf * 1e6, 4)}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(p, ms, W, budget_s):
    """The fp64 oracle (as it stands) on the host cores: repeated verify steps
    (one oracle call per M) until about 2/3 of budget_s is spent with the BLAS
    pool at its default size, then at least three steps with it pinned to one
    thread.  Per M the median call time is taken; the value is the weight
    bytes of one step over the sum of those medians."""
    sys.path.insert(0, ROOT)
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits
    s = p.shape

    def blas_threads():
        return max([i.get("num_threads", 1) for i in threadpool_info()
                    if i.get("user_api") == "blas"] or [1])

    def run(budget, min_steps):
        times = {M: [] for M in ms}
        t0 = time.perf_counter()
        steps = 0
        while steps < min_steps or time.perf_counter() - t0 < budget:
            for M in ms:
                c0 = time.perf_counter()
                if s.fmt is not None:
                    oracle.qgemv_fp_reference(p.codes, p.scales, p.x, M, s.N, s.K, s.fmt)
                else:
                    oracle.qgemv_reference(p.codes, p.scales, p.biases, p.x, M, s.N, s.K, s.bits,
                                           s.group_size)
                times[M].append(time.perf_counter() - c0)
            steps += 1
        med = {M: statistics.median(v) for M, v in times.items()}
        return {"GBps": round(W * len(ms) / sum(med.values()) / 1e9, 4), "steps": steps,
                "median_ms_per_call": {str(M): round(v * 1e3, 2) for M, v in med.items()},
                "wall_s": round(time.perf_counter() - t0, 1)}

    threads = blas_threads()
    blas = [{"library": i.get("internal_api"), "version": i.get("version"),
             "threading_layer": i.get("threading_layer"), "num_threads": i.get("num_threads")}
            for i in threadpool_info() if i.get("user_api") == "blas"]
    multi = run(budget_s * 2 / 3, 3)
    with threadpool_limits(limits=1, user_api="blas"):
        single = run(0.0, 3)
    return {"value": multi["GBps"], "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{multi['steps']} verify steps (one oracle call per M in {ms}) of {s.name}; "
                      f"median call time per M; numpy fp64 unpack + dequantize + BLAS matmul",
            "median_ms_per_call": multi["median_ms_per_call"], "wall_s": multi["wall_s"],
            "one_thread": single, "cpu_count": os.cpu_count(), "cpu_model": cpu_model(), "blas": blas}


if __name__ == "__main__":
    main()
