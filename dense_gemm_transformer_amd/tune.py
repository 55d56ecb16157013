"""Measure candidate plans per shape and write the dispatch table.

    python -m dense_gemm_transformer_amd.tune [--out csrc/dispatch_table.inc] [--rounds 5]

For every workload shape (the five linear-layer workloads and the backward
GEMMs of a GPT-2-small layer) each candidate
plan — stream and tiled configurations, with and without split-K — runs in
paired rounds: one timing of every candidate per round, the round order
rotating, the median over rounds kept ("compare only within one window", the
paired measurements of "Optimizing a GPT-2-class transformer on a GPU", Act V).
Each timing replays a CUDA graph of back-to-back launches, so host launch
overhead does not hide microsecond kernels.  A candidate whose output differs
from the planner's default plan by more than the parity tolerance is dropped.
The winner of each shape becomes one row of ``csrc/dispatch_table.inc``; with
``--only`` the rows of the shapes not measured are kept from the existing table.
The table keys on the kernel epilogue (bias, GELU) only, so a residual case is
timed without its residual: the flag adds one read of Y to the same kernel.
"""

from __future__ import annotations

import argparse
import json
import os
import statistics
import sys

import numpy as np

from . import inputs

HERE = os.path.dirname(os.path.abspath(__file__))
TABLE = os.path.join(HERE, "csrc", "dispatch_table.inc")


def workload_cases():
    cases = [inputs.workload_fp32_linear_128x768(), inputs.workload_fp16_narrow()]
    cases += inputs.workload_gpt2_layer(M=128, dtype="f32")
    cases += [inputs.workload_square(dtype="f32"), inputs.workload_square(dtype="bf16")]
    cases += inputs.workload_gpt2_layer(M=8192, dtype="f32") + inputs.workload_gpt2_layer(M=8192, dtype="bf16")
    cases += inputs.workload_gpt2_backward(dtype="f32") + inputs.workload_gpt2_backward(dtype="bf16")
    return cases


_DT = {"f32": 0, "f16": 1, "bf16": 2}
_LAY = {"NK": 0, "KN": 1, "AT_NK": 2, "AT_KN": 3}


def table_row(M, N, K, in_dtype, out_dtype, layout, epi, v, tile, split, comment) -> str:
    return (f"{{{M}, {N}, {K}, {_DT[in_dtype]}, {_DT[out_dtype]}, {_LAY[layout]}, {epi}u, {v}, {tile}, "
            f"{split}}},  // {comment}")


def existing_rows(path):
    """Rows of a table file as {shape key: line}; the sentinel and comments are skipped."""
    rows = {}
    if not os.path.exists(path):
        return rows
    for line in open(path):
        line = line.strip()
        if not line.startswith("{"):
            continue
        fields = [f.strip().rstrip("u") for f in line[1:line.index("}")].split(",")]
        key = tuple(int(f) for f in fields[:7])
        if key[0] >= 1:
            rows[key] = line
    return rows


def candidates(case, tlgemm):
    """(variant, tile, split) triples the planner accepts for this shape."""
    out = []
    opts = []
    if case.layout == "NK" and case.M <= 256:
        for tile in range(1, 6):
            opts += [(tlgemm.VARIANT_STREAM, tile, 0), (tlgemm.VARIANT_STREAM, tile, 1)]
    for tile in range(1, 6):
        for split in (1, 2, 4, 8):
            opts.append((tlgemm.VARIANT_TILED, tile, split))
    for v, tile, split in opts:
        try:
            p = tlgemm.Plan.create(case.M, case.N, case.K, case.in_dtype, case.out_dtype, case.layout,
                                   case.b is not None, case.gelu, v, split, tile)
        except tlgemm.TlgError:
            continue
        key = p.describe()
        if all(key != o[3] for o in out):
            out.append((v, tile, split, key, p))
        else:
            p.close()
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--out", default=TABLE)
    ap.add_argument("--rounds", type=int, default=5)
    ap.add_argument("--launches", type=int, default=20, help="launches per captured graph")
    ap.add_argument("--only", default="", help="comma-separated substrings: tune only workloads naming one")
    ap.add_argument("--jsonl", default="", help="append every measurement here")
    args = ap.parse_args(argv)

    import torch

    from . import tlgemm

    dev = torch.device("cuda:0")

    def put(a, dt):
        if dt == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    rows = []
    log = open(args.jsonl, "a") if args.jsonl else None
    for case in workload_cases():
        if args.only and not any(o in case.name for o in args.only.split(",")):
            continue
        X, W = put(case.X, case.in_dtype), put(case.W, case.in_dtype)
        b = None if case.b is None else put(case.b, case.in_dtype)
        cands = candidates(case, tlgemm)
        ydt = tlgemm.torch_dtype(case.out_dtype)
        ref_plan = tlgemm.Plan.create(case.M, case.N, case.K, case.in_dtype, case.out_dtype, case.layout,
                                      case.b is not None, case.gelu)
        ref = tlgemm.run(ref_plan, X, W, b).float()
        tol = 1e-5 if case.in_dtype == "f32" else 1e-2
        scale = ref.abs().max().item() or 1.0
        graphs = []
        for v, tile, split, key, p in cands:
            Y = torch.empty((case.M, case.N), dtype=ydt, device=dev)
            ws = torch.zeros(max(p.workspace_size, 1), dtype=torch.uint8, device=dev)
            args_ = (X.data_ptr(), W.data_ptr(), 0 if b is None else b.data_ptr(), Y.data_ptr(),
                     ws.data_ptr() if p.workspace_size else 0, p.workspace_size)
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                p.run_ptrs(*args_, s.cuda_stream)
            s.synchronize()
            if (Y.float() - ref).abs().max().item() > tol * scale:
                print(f"# dropped (parity): {key}", file=sys.stderr)
                continue
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                for _ in range(args.launches):
                    p.run_ptrs(*args_, s.cuda_stream)
            g.replay()
            torch.cuda.synchronize()
            graphs.append(((v, tile, split, key), g, Y, ws))
        times = {c[0]: [] for c in graphs}
        for rnd in range(args.rounds):
            order = graphs[rnd % len(graphs):] + graphs[:rnd % len(graphs)]
            for cand, g, _, _ in order:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                g.replay()
                e1.record()
                torch.cuda.synchronize()
                times[cand].append(e0.elapsed_time(e1) * 1e3 / args.launches)
        med = {c: statistics.median(t) for c, t in times.items()}
        best = min(med, key=med.get)
        for c, m in sorted(med.items(), key=lambda kv: kv[1]):
            line = {"workload": case.name, "plan": c[3], "us": round(m, 3),
                    "tflops": round(case.flops / m / 1e6, 2), "best": c == best}
            print(json.dumps(line), flush=True)
            if log:
                log.write(json.dumps(line) + "\n")
        v, tile, split, key = best
        p_best = tlgemm.Plan.create(case.M, case.N, case.K, case.in_dtype, case.out_dtype, case.layout,
                                    case.b is not None, case.gelu, v, split, tile)
        info = p_best.info
        epi = (1 if case.b is not None else 0) | (2 if case.gelu else 0)
        rows.append((case, v, tile - 1, info.split_k, epi, med[best], p_best.describe()))
        del graphs
        torch.cuda.synchronize()

    if rows and args.out:
        merged = existing_rows(args.out) if args.only else {}
        for case, v, tile, split, epi, us, desc in rows:
            key = (case.M, case.N, case.K, _DT[case.in_dtype], _DT[case.out_dtype], _LAY[case.layout], epi)
            merged[key] = table_row(case.M, case.N, case.K, case.in_dtype, case.out_dtype, case.layout, epi,
                                    v, tile, split, f"{case.name}: {us:.2f} us")
        with open(args.out, "w") as f:
            f.write("// Measured per-shape routing: {M, N, K, in_dt, out_dt, layout, epi, variant, tile, split}.\n")
            f.write("// Written by `python -m dense_gemm_transformer_amd.tune` on one MI355X: the fastest\n")
            f.write("// candidate of paired rounds, each timing a graph replay of back-to-back launches.\n")
            f.write("{0, 0, 0, 0, 0, 0, 0u, 0, 0, 0},  // sentinel (matches no shape: M >= 1 is enforced)\n")
            for line in merged.values():
                f.write(line + "\n")
        print(f"# wrote {len(merged)} rows ({len(rows)} measured) to {args.out}", file=sys.stderr)
    return 0


if __name__ == "__main__":
    sys.exit(main())
