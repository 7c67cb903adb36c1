"""Dispatcher calibration: forced-path sweep of the dot and MFMA paths.

    python -m few_row_quantized_amd.calibrate --out select_sweep.json
    python -m few_row_quantized_amd.calibrate --emit-header select_sweep.json

The first form runs on the GPU: for every workload shape (the square and
FFN-up projections, the 2-bit 27B-class FFN and the seven projections of one
27B-class decoder layer) and every M = 1..16 it times each path that supports
the shape, as the pages recommend for this decision (MLX quantized_matmul
small-M verify kernels, Facts: forced-path qmv vs qmm sweeps; dependent chains
rather than independent queue-batched calls).  Every launch reads its weights
from the next copy of a rotating pool larger than the caches; times are
averages over a HIP-graph chain of launches.

The second form turns a sweep into csrc/qgemv_select_table.h: for each
(bits, group size, N class, K class) the set of M at which the MFMA path was
faster, as a 16-bit mask.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(PKG))

from few_row_quantized_amd import accounting, synth  # noqa: E402

# Table keys of the block-scaled FP formats: bits = 100 + format code.
FP_CODES = {"mxfp4": 1, "nvfp4": 2, "mxfp8": 3}

# Shape classes of the table (boundaries in elements).
N_CLASSES = [(0, 2048), (2048, 8192), (8192, 1 << 30)]
K_CLASSES = [(0, 8192), (8192, 1 << 30)]


def n_class(N: int) -> int:
    return next(i for i, (lo, hi) in enumerate(N_CLASSES) if lo < N <= hi)


def k_class(K: int) -> int:
    return next(i for i, (lo, hi) in enumerate(K_CLASSES) if lo < K <= hi)


def sweep(names, ms, chain: int, pool_mib: int, log=print):
    import numpy as np
    import torch
    from few_row_quantized_amd import qgemv as q

    def timed(fn, n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(n):
                fn()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / (2 * n)

    rows = []
    for name in names:
        s = synth.WORKLOADS[name]
        p = synth.make_problem(s, m_max=16)
        fp = s.fmt is not None
        W = (accounting.fp_weight_bytes(s.N, s.K, s.bits, s.group_size) if fp else
             accounting.weight_bytes(s.N, s.K, s.bits, s.group_size))
        P = max(2, math.ceil(pool_mib * 2 ** 20 / W))
        codes = torch.from_numpy(p.codes).cuda().unsqueeze(0).repeat(P, 1, 1)
        sc = torch.from_numpy(p.scales if fp else p.scales.view(np.int16)).cuda().unsqueeze(0).repeat(P, 1, 1)
        bi = None if fp else torch.from_numpy(p.biases.view(np.int16)).cuda().unsqueeze(0).repeat(P, 1, 1)
        x = torch.from_numpy(p.x.view(np.int16)).cuda()
        y = torch.empty((16, s.N), dtype=torch.float32, device="cuda")
        for M in ms:
            rec = {"workload": name, "K": s.K, "N": s.N, "bits": s.bits, "group_size": s.group_size,
                   "M": M, "weight_bytes": W}
            if fp:
                rec["fmt"] = s.fmt
            for path in ("dot", "mfma"):
                if fp:
                    if not q.qgemv_path_supported_fp(path, M, s.N, s.K, s.fmt):
                        continue
                elif not q.qgemv_path_supported(path, M, s.N, s.K, s.bits, s.group_size):
                    continue
                ctr = [0]

                def one():
                    i = ctr[0] % P
                    ctr[0] += 1
                    if fp:
                        q.qgemv_run_path_fp(path, codes[i], sc[i], x, None, y, M, s.N, s.K, s.fmt)
                    else:
                        q.qgemv_run_path(path, codes[i], sc[i], bi[i], x, y, M, s.N, s.K, s.bits,
                                         s.group_size)

                one()
                torch.cuda.synchronize()
                rec[f"{path}_us"] = round(timed(one, chain) * 1e6, 4)
            rows.append(rec)
            log(json.dumps(rec))
        del codes, sc, bi
        torch.cuda.empty_cache()
    return rows


def table_from_sweep(rows):
    """(bits, gs, n_class, k_class) -> 16-bit mask of M where MFMA was faster.

    Several shapes in one class: MFMA where the geometric mean over them of
    t_mfma / t_dot is below 1 (the choice that costs least in relative time
    summed over the class), so a large win on one shape outweighs a small
    loss on another."""
    ratios = {}
    for r in rows:
        if "mfma_us" not in r or "dot_us" not in r:
            continue
        # FP formats are keyed by 100 + format code, group size 0
        key = ((100 + FP_CODES[r["fmt"]], 0) if "fmt" in r else (r["bits"], r["group_size"])) + (
            n_class(r["N"]), k_class(r["K"]))
        ratios.setdefault(key, {}).setdefault(r["M"], []).append(math.log(r["mfma_us"] / r["dot_us"]))
    table = {}
    for key, per_m in ratios.items():
        mask = 0
        for M, v in per_m.items():
            if sum(v) < 0:
                mask |= 1 << (M - 1)
        table[key] = mask
    return table


def emit_header(table, source: str) -> str:
    lines = [
        "// Dot-vs-MFMA choice used by qgemv_select -- generated by",
        "// `python -m few_row_quantized_amd.calibrate --emit-header " + source + "`;",
        "// do not edit by hand.",
        "//",
        "// The pages show that the row count where a matrix-unit kernel overtakes the",
        "// mat-vec kernel depends on the format, the shape and the device (few-row MMA",
        "// PR, Overview: per-type start rows tuned on one GPU and reached later on",
        "// another; MLX page, Facts: per-architecture batch limits and bit-width",
        "// gating).  This table is measured on MI355X: for each (bits, group size,",
        "// N class, K class) bit M-1 of the mask is set when the MFMA path was the",
        "// faster one for M activation rows in a forced-path sweep.  Block-scaled",
        "// FP formats are keyed by bits = 100 + format (1 mxfp4, 2 nvfp4, 3 mxfp8).",
        "#pragma once",
        "",
        "#include <stdint.h>",
        "",
        "namespace qgemv {",
        "",
        "struct SelectEntry {",
        "  int bits, group_size, n_class, k_class;",
        "  uint32_t mfma_mask;",
        "};",
        "",
        "// N classes: " + ", ".join(f"({lo}, {hi}]" for lo, hi in N_CLASSES),
        "// K classes: " + ", ".join(f"({lo}, {hi}]" for lo, hi in K_CLASSES),
        "inline int select_n_class(int N) { return N <= %d ? 0 : (N <= %d ? 1 : 2); }"
        % (N_CLASSES[0][1], N_CLASSES[1][1]),
        "inline int select_k_class(int K) { return K <= %d ? 0 : 1; }" % K_CLASSES[0][1],
        "",
        "constexpr SelectEntry kSelectTable[] = {",
    ]
    for (bits, gs, nc, kc), mask in sorted(table.items()):
        lines.append(f"    {{{bits}, {gs}, {nc}, {kc}, 0x{mask:04x}u}},")
    lines += [
        "};",
        "",
        "}  // namespace qgemv",
        "",
    ]
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default="select_sweep.json")
    ap.add_argument("--workloads", default=None,
                    help="comma list; default: all but the tiny one and the FP formats; 'fp': the FP formats")
    ap.add_argument("--chain", type=int, default=200)
    ap.add_argument("--pool-mib", type=int, default=1024)
    ap.add_argument("--emit-header", default=None, metavar="SWEEP_JSON",
                    help="write csrc/qgemv_select_table.h from a sweep file")
    args = ap.parse_args()
    if args.emit_header:
        rows = json.load(open(args.emit_header))["rows"]
        hdr = emit_header(table_from_sweep(rows), os.path.relpath(os.path.abspath(args.emit_header), os.path.dirname(PKG)))
        path = os.path.join(PKG, "csrc", "qgemv_select_table.h")
        open(path, "w").write(hdr)
        print(f"wrote {path}")
        return
    if args.workloads == "fp":
        names = [n for n, w in synth.WORKLOADS.items() if w.fmt is not None]
    else:
        names = (args.workloads.split(",") if args.workloads else
                 [n for n, w in synth.WORKLOADS.items() if not n.startswith("tiny") and w.fmt is None])
    t0 = time.time()
    rows = sweep(names, list(range(1, 17)), args.chain, args.pool_mib,
                 log=lambda m: print(m, flush=True))
    json.dump({"rows": rows, "seconds": round(time.time() - t0, 1)}, open(args.out, "w"), indent=0)
    print(f"wrote {args.out} ({len(rows)} rows)", flush=True)


if __name__ == "__main__":
    main()
