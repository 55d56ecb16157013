"""Search the plan space per shape and write the dispatch table.

    python -m dense_gemm_transformer_amd.tune [--out csrc/dispatch_table.inc] [--rounds 7]
        [--budget 6] [--explore 2] [--exhaustive] [--cold] [--only a,b] [--jsonl log] [--report md]

The search loop of "Optimizing a GPT-2-class transformer on a GPU" (Act V),
with its cost model and rules in ``search.py``.  For every workload shape (the
five linear-layer workloads and the backward GEMMs of a GPT-2-small layer):

1. Propose: every (variant, tile, split) the planner accepts, minus the
   candidates the hard constraints exclude.
2. Stop early when the incumbent (the planner's current choice for the shape)
   already runs within ``--stop-eff`` of the physical floor.
3. Predict each candidate's time (roofline prior × the residual regression
   fitted on every shape measured so far) and measure the ``--budget`` best
   predictions, the ``--explore`` candidates the model is least sure of, and
   the incumbent, in paired rounds: one timing of each per round, the order
   rotating, all in one window.  Each timing replays a graph of back-to-back
   launches, so host launch overhead does not hide microsecond kernels; with
   ``--cold`` the launches rotate over copies of the operands larger than the
   Infinity Cache, as a pass over distinct layers reads them.  A
   candidate whose output differs from the incumbent's by more than the
   parity tolerance is dropped.
4. Select: the fastest candidate replaces the incumbent only if the paired
   rounds say so (``search.decide``); score = efficiency against the floor.
5. Learn: add the measurements to the regression and refit.

The chosen plan of each shape becomes one row of ``csrc/dispatch_table.inc``;
with ``--only`` the rows of the shapes not searched are kept.  The table keys
on the kernel epilogue (bias, GELU) only, so a residual case is timed without
its residual: the flag adds one read of Y to the same kernel.  The residual
report (the regression's coefficients) closes the run.
"""

from __future__ import annotations

import argparse
import json
import os
import statistics
import sys

import numpy as np

from . import inputs, search

HERE = os.path.dirname(os.path.abspath(__file__))
TABLE = os.path.join(HERE, "csrc", "dispatch_table.inc")
# Length of each variant's tile list (for 16-bit inputs, the longer tiled list):
# the options a search walks.  A CPU test checks them against the planner.
STREAM_OPTIONS = 15
TILED_OPTIONS = 13


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
    """(variant, tile, split, key, plan) for every configuration the planner accepts for this shape."""
    out = []
    opts = []
    if case.layout == "NK" and case.M <= 256:
        for tile in range(1, STREAM_OPTIONS + 1):
            # the automatic split, none, and 2 or 4 (the automatic split gives the
            # pipelined options one chunk per split, which leaves nothing to overlap)
            opts += [(tlgemm.VARIANT_STREAM, tile, split) for split in (0, 1, 2, 4)]
    for tile in range(1, TILED_OPTIONS + 1):  # past the dtype's tile list the planner refuses, and the option is skipped
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


def config_of(plan, key) -> search.Config:
    i = plan.info
    return search.Config(i.variant, i.tile_m, i.tile_n, i.tile_k, i.split_k, i.threads, i.workgroups,
                         i.launches, key)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--out", default=TABLE)
    ap.add_argument("--rounds", type=int, default=7)
    ap.add_argument("--launches", type=int, default=20, help="launches per captured graph")
    ap.add_argument("--cold", action="store_true",
                    help="rotate the launches over copies of X and W totalling over 512 MiB (more than the "
                         "Infinity Cache), so that operands come from HBM as in a pass over distinct layers")
    ap.add_argument("--budget", type=int, default=6, help="candidates measured by best prediction")
    ap.add_argument("--explore", type=int, default=2, help="candidates measured by largest model uncertainty")
    ap.add_argument("--exhaustive", action="store_true", help="measure every allowed candidate")
    ap.add_argument("--margin", type=float, default=0.01, help="paired gain a challenger needs over the incumbent")
    ap.add_argument("--stop-eff", type=float, default=0.9,
                    help="skip shapes whose incumbent reaches this efficiency against the physical floor")
    ap.add_argument("--only", default="", help="comma-separated substrings: search only workloads naming one")
    ap.add_argument("--jsonl", default="", help="append every measurement here")
    ap.add_argument("--report", default="", help="write a markdown summary and the residual report here")
    args = ap.parse_args(argv)

    import torch

    from . import tlgemm

    dev = torch.device("cuda:0")

    def put(a, dt):
        if dt == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    model = search.ResidualModel()
    rows, summary = [], []
    log = open(args.jsonl, "a") if args.jsonl else None

    def emit(line):
        print(json.dumps(line), flush=True)
        if log:
            log.write(json.dumps(line) + "\n")

    for case in workload_cases():
        if args.only and not any(o in case.name for o in args.only.split(",")):
            continue
        shape = search.Shape(case.M, case.N, case.K, case.in_dtype, case.out_dtype)
        X, W = put(case.X, case.in_dtype), put(case.W, case.in_dtype)
        b = None if case.b is None else put(case.b, case.in_dtype)
        # operand copies the captured launches rotate over (one: warm, the same operands every launch)
        ncopy = 1
        if args.cold:
            nbytes = X.numel() * X.element_size() + W.numel() * W.element_size()
            ncopy = min(64, max(2, -(-(512 << 20) // nbytes)))
        XW = [(X, W)] + [(X.clone(), W.clone()) for _ in range(ncopy - 1)]
        ydt = tlgemm.torch_dtype(case.out_dtype)
        inc_plan = tlgemm.Plan.create(case.M, case.N, case.K, case.in_dtype, case.out_dtype, case.layout,
                                      case.b is not None, case.gelu)
        inc_key = inc_plan.describe()
        cands = candidates(case, tlgemm)
        configs = {key: config_of(p, key) for _, _, _, key, p in cands}
        by_key = {key: (v, tile, split, p) for v, tile, split, key, p in cands}
        if inc_key not in by_key:  # the incumbent is always a candidate
            by_key[inc_key] = (inc_plan.info.variant, 0, 0, inc_plan)
            configs[inc_key] = config_of(inc_plan, inc_key)
        ref = tlgemm.run(inc_plan, X, W, b).float()
        tol = 1e-5 if case.in_dtype == "f32" else 1e-2
        scale = ref.abs().max().item() or 1.0

        def build(key):
            p = by_key[key][3]
            Y = torch.empty((case.M, case.N), dtype=ydt, device=dev)
            ws = torch.zeros(max(p.workspace_size, 1), dtype=torch.uint8, device=dev)
            args_ = (X.data_ptr(), W.data_ptr(), 0 if b is None else b.data_ptr(), Y.data_ptr(),
                     ws.data_ptr() if p.workspace_size else 0, p.workspace_size)
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())  # Y, ws and the inputs come from the default stream
            with torch.cuda.stream(s):
                p.run_ptrs(*args_, s.cuda_stream)
            s.synchronize()
            if (Y.float() - ref).abs().max().item() > tol * scale:
                print(f"# dropped (parity): {key}", file=sys.stderr)
                return None
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                for i in range(args.launches):
                    Xi, Wi = XW[i % ncopy]
                    p.run_ptrs(Xi.data_ptr(), Wi.data_ptr(), *args_[2:], s.cuda_stream)
            g.replay()
            torch.cuda.synchronize()
            return (key, g, Y, ws)

        def time_graph(g):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e-3 / args.launches  # seconds per launch

        # Port 2's stopping rule: an incumbent at the floor is not searched.
        inc = build(inc_key)
        inc_s = statistics.median(time_graph(inc[1]) for _ in range(3))
        inc_eff = search.efficiency(shape, inc_s)
        if inc_eff >= args.stop_eff:
            emit({"workload": case.name, "plan": inc_key, "us": round(inc_s * 1e6, 3),
                  "efficiency": round(inc_eff, 4), "best": True, "stopped": True})
            summary.append((case.name, inc_key, inc_s, inc_eff, 1, "kept: at the floor"))
            rows.append((case, inc_plan, inc_s, tile_index(by_key[inc_key])))
            del inc
            continue

        allowed = search.constrained(shape, list(configs.values()))
        if args.exhaustive:
            picked = allowed + ([configs[inc_key]] if all(c.key != inc_key for c in allowed) else [])
        else:
            picked = search.choose(shape, allowed, model, args.budget, args.explore, inc_key)
        graphs = [inc] + [g for g in (build(c.key) for c in picked if c.key != inc_key) if g is not None]
        times = {gk[0]: [] for gk in graphs}
        for rnd in range(args.rounds):
            order = graphs[rnd % len(graphs):] + graphs[:rnd % len(graphs)]
            for key, g, _, _ in order:
                times[key].append(time_graph(g))
        med = {k: statistics.median(t) for k, t in times.items()}
        for k, m in med.items():
            f = search.features(shape, configs[k])
            model.add(f, search.prior_s(shape, f), m)
        best = min(med, key=med.get)
        dec = search.decide(times[inc_key], times[best], args.margin) if best != inc_key else None
        chosen = inc_key if dec is None or dec.keep_incumbent else best
        for k, m in sorted(med.items(), key=lambda kv: kv[1]):
            f = search.features(shape, configs[k])
            pr = search.prior_s(shape, f)
            emit({"workload": case.name, "plan": k, "us": round(m * 1e6, 3), "tflops": round(case.flops / m / 1e12, 2),
                  "efficiency": round(search.efficiency(shape, m), 4), "prior_us": round(pr * 1e6, 2),
                  "predicted_us": round(model.predict_s(f, pr) * 1e6, 2), "best": k == chosen,
                  "incumbent": k == inc_key})
        model.fit()
        verdict = "kept: no challenger" if dec is None else ("kept: " if dec.keep_incumbent else "replaced: ") + dec.reason
        summary.append((case.name, chosen, med[chosen], search.efficiency(shape, med[chosen]), len(graphs), verdict))
        rows.append((case, by_key[chosen][3], med[chosen], tile_index(by_key[chosen])))
        del graphs
        torch.cuda.synchronize()

    report = model.report()
    print("# residual report (log(measured/prior) on features):", file=sys.stderr)
    for name, coef, verdict in report:
        print(f"#   {name:34s} {coef:+.3f}  {verdict}", file=sys.stderr)

    if rows and args.out:
        merged = existing_rows(args.out) if args.only else {}
        for case, p, s, tile in rows:
            i = p.info
            epi = (1 if case.b is not None else 0) | (2 if case.gelu else 0)
            key = (case.M, case.N, case.K, _DT[case.in_dtype], _DT[case.out_dtype], _LAY[case.layout], epi)
            merged[key] = table_row(case.M, case.N, case.K, case.in_dtype, case.out_dtype, case.layout, epi,
                                    i.variant, tile, i.split_k, f"{case.name}: {s * 1e6:.2f} us")
        with open(args.out, "w") as f:
            f.write("// Measured per-shape routing: {M, N, K, in_dt, out_dt, layout, epi, variant, tile, split}.\n")
            f.write("// Written by `python -m dense_gemm_transformer_amd.tune` on one MI355X: the plan its\n")
            f.write("// search kept per shape, timed as graph replays of back-to-back launches.\n")
            f.write("{0, 0, 0, 0, 0, 0, 0u, 0, 0, 0},  // sentinel (matches no shape: M >= 1 is enforced)\n")
            for line in merged.values():
                f.write(line + "\n")
        print(f"# wrote {len(merged)} rows ({len(rows)} searched) to {args.out}", file=sys.stderr)

    if args.report:
        with open(args.report, "w") as f:
            f.write("| workload | kept plan | µs | efficiency vs floor | measured | decision |\n|---|---|---|---|---|---|\n")
            for name, key, s, eff, n, verdict in summary:
                f.write(f"| {name} | `{key}` | {s * 1e6:.2f} | {eff:.3f} | {n} | {verdict} |\n")
            f.write("\nResidual report: coefficients of log(measured / prior) on the features "
                    f"({len(model.y)} measurements).\n\n| feature | coefficient | verdict |\n|---|---|---|\n")
            for name, coef, verdict in report:
                f.write(f"| {name} | {coef:+.3f} | {verdict} |\n")
    return 0


def tile_index(entry) -> int:
    """Index of a candidate's tile in its variant's tile list (what a table row stores)."""
    v, tile, split, plan = entry
    return tile - 1 if tile > 0 else table_tile(plan)


def table_tile(plan) -> int:
    """The tile index that reproduces ``plan`` (for an incumbent no candidate option produced)."""
    from . import tlgemm

    i = plan.info
    for t in range(1, max(TILED_OPTIONS, STREAM_OPTIONS) + 1):
        try:
            q = tlgemm.Plan.create(plan.M, plan.N, plan.K, plan.in_dtype, plan.out_dtype, plan.layout,
                                   bool(plan.epi_flags & 1), bool(plan.epi_flags & 2), i.variant, max(i.split_k, 1)
                                   if i.variant == tlgemm.VARIANT_TILED else i.split_k, t)
        except tlgemm.TlgError:
            continue
        same = q.describe() == plan.describe()
        q.close()
        if same:
            return t - 1
    raise RuntimeError(f"no tile index reproduces {plan.describe()}")


if __name__ == "__main__":
    sys.exit(main())
