#!/usr/bin/env python3
"""Benchmark of the transformer linear-layer GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--ramp-ms R] [--no-cpu-baseline]

A step is one call of the library on the square fp32 GEMM C = A·B with
M = N = K = 4096 and row-major A and B (warm operands).  Its throughput in
TFLOP/s is ``value``.  The same run also times the narrow fp16 linear
Y = X·Wᵀ with X 16×4096 and W 4096×4096 out×in, fp16 output, with cold
weights: the launches rotate through 16 identical copies of W (512 MiB, more
than the 256 MB Infinity Cache plus L2), as on "One multiply, one RTX 5090,
eight kernels" ("Where the time goes").  That result is reported in µs and
GB/s under ``narrow_fp16``.  Both results carry a parity verdict against
the CPU oracle on sampled outputs, and both come with their roofline
fraction: MFMA fp32 peak 157.3 TFLOP/s for the square GEMM, HBM 8 TB/s for
the narrow one.

Beside them (skipped with ``--no-extra``): the achievable ceilings from
probe kernels (launch floor, plain 32 MiB read cold and warm, MFMA issue
rate); the fp32 linear 128×768×768 + bias warm and cold; the four GPT-2-small
linears at M = 128 (fp32), each warm and as a layer warm and cold; and one
pass of the batched GPT-2-small stack at M = 8192 (12 layers × 4 linears, 48
launches) in fp32 and bf16, with tokens/s; and the backward GEMMs of one
GPT-2-small layer at 8192 tokens (dX with the [K][N] weight layout, dW with the
transposed first operand accumulated onto the previous gradient); LayerNorm and
fused causal attention at GPT-2-small size; and the GPT-2-small forward through
12 blocks composed from all of them (tokens/s).

Every timed region is preceded by R milliseconds (default 300) of untimed
back-to-back launches of its own work, then (for the square GEMMs) the W
warmup steps: from idle the core clock needs tens of milliseconds of load to
come up, and the bench measures the loaded clock (``clock_ramp_ms`` in the
output line).

The oracle (plain C, double accumulation) is timed on this host's cores on
a bounded row sample of the square workload and reported as
``cpu_baseline``; it is a reference point, not a target.

Prints one JSON line.  ``--gpus`` above 1 exits with a message: the library
runs on one GPU.
"""

from __future__ import annotations

import argparse
import glob
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "TFLOP/s (% MFMA peak) @4096³ fp32; µs + HBM GB/s @16×4096×4096 fp16"

# Bytes each kernel moved between L2 and memory per launch, from rocprofv3
# FETCH_SIZE and WRITE_SIZE passes over `bench.py --steps 3 --warmup 1
# --narrow-launches 32 --no-cpu-baseline --no-parity --no-extra --no-vendor --ramp-ms 0`, summarised
# by `bench.py --pmc-summary` (the HBM-traffic profile under profiles/).
# FETCH_SIZE is scaled by 1.998 and WRITE_SIZE by 1.0: the factors that make
# the same counters read 32 MiB for the run's 32 MiB device-to-device copies.
# Each entry holds the hash of the kernel sources and the tile it was taken on;
# after a change to either the figure no longer applies and the bench reports null.
FETCH_SCALE, WRITE_SCALE = 1.998, 1.0
TRAFFIC = {
    "tiled_f32": {"sources": ("common.h", "tiled.h"), "sha": "6f4660e0ad36dce1",
                  "tile": "256x256x16", "fetch_kib": 196687.0, "write_kib": 65536.0},
    "stream_f16": {"sources": ("common.h", "stream.h"), "sha": "7278d7ba9ee58e13",
                   "tile": "16x16x4096", "fetch_kib": 16919.0, "write_kib": 128.0},
}


def measured_traffic(key: str, tile: str):
    """HBM bytes per launch for a kernel, or None if its sources or tile changed since the counters were taken."""
    import hashlib

    rec = TRAFFIC[key]
    h = hashlib.sha256()
    for name in rec["sources"]:
        with open(os.path.join(ROOT, "dense_gemm_transformer_amd", "csrc", "kernels", name), "rb") as f:
            h.update(f.read())
    if h.hexdigest()[:16] != rec["sha"] or tile != rec["tile"]:
        return None
    return int((rec["fetch_kib"] * FETCH_SCALE + rec["write_kib"] * WRITE_SCALE) * 1024)
def tile_str(plan) -> str:
    i = plan.info
    return f"{i.tile_m}x{i.tile_n}x{i.tile_k}"


PEAK_F32_TFLOPS = 157.3      # MI355X dense fp32 matrix
PEAK_BF16_TFLOPS = 2516.6    # MI355X dense bf16/fp16 matrix
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
PEAK_SCLK_MHZ = 2400.0       # the core clock the datasheet peaks assume
COLD_COPIES = 16


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def read_clocks(torch):
    """Current sclk/mclk levels of this process's GPU, read from the amdgpu driver's sysfs tables
    (the level marked '*'), matched to the device by PCI address; None if unavailable.  No
    subprocess: a helper program started under a profiler would inherit its preloaded library."""
    try:
        pr = torch.cuda.get_device_properties(0)
        bdf = f"{pr.pci_domain_id:04x}:{pr.pci_bus_id:02x}:{pr.pci_device_id:02x}."
        for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
            if not os.path.basename(os.path.realpath(dev)).startswith(bdf):
                continue
            out = {}
            for clk in ("sclk", "mclk"):
                with open(os.path.join(dev, f"pp_dpm_{clk}")) as f:
                    cur = [ln.strip() for ln in f if ln.rstrip().endswith("*")]
                out[clk] = cur[0] if cur else None
            return out
    except Exception:
        return None
    return None


RAMP_MS = 300.0  # default --ramp-ms


def ramp(fn, stream, min_ms: float = None) -> float:
    """Run ``fn(i)`` back to back, untimed, until at least ``min_ms`` of GPU time has passed; returns that time.

    From idle (the host generating inputs, the oracle checking a sample) the
    core clock takes tens of milliseconds of load to come up: the square bf16
    4096³ GEMM measured 133–137 µs per launch after 10 launches from a
    second of idle and 112 µs after 400 (fp32: 936–945 against 915–918 µs).
    Every timed region of this bench is preceded by such a ramp of its own
    work, so that it measures the loaded clock, as a busy GPU runs.
    """
    import torch

    min_ms = RAMP_MS if min_ms is None else min_ms
    spent, n, i = 0.0, 1, 0
    while spent < min_ms:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            fn(i)
            i += 1
        b.record(stream)
        torch.cuda.synchronize()
        spent += a.elapsed_time(b)
        n = min(2 * n, 4096)
    return spent


def l2_roofline(ceil, plan, case, ms: float) -> dict:
    """The square GEMM against the on-chip read rate: every workgroup streams a BM-row panel of A and a BN-column
    panel of B through its CU, so one launch moves es·K·(M·N/BN + N·M/BM) bytes from L2 to the CUs; that over
    the launch time, against the rate of the ceiling probe that re-reads L2-resident blocks on every CU."""
    if not ceil or "read_l2_GB/s" not in ceil:
        return {}
    i = plan.info
    es = 4 if case.in_dtype == "f32" else 2
    nbytes = es * case.K * (case.M * case.N // i.tile_n + case.N * case.M // i.tile_m)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"l2_to_cu": {"bytes_per_launch": nbytes, "GB/s": round(gbs, 1), "ceiling_GB/s": ceil["read_l2_GB/s"],
                         "frac": round(gbs / ceil["read_l2_GB/s"], 4)}}


def time_launches(fn, n: int, stream) -> float:
    """Average ms per call of ``fn(i)`` over n back-to-back calls, HIP events on ``stream``."""
    import torch

    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(n):
        fn(i)
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / n


def vendor_entry(call: str, vendor_ms: float, ours_ms: float) -> dict:
    """One row of the vendor-library context: its time beside this library's on the same inputs and stream."""
    return {"call": call, "us": round(vendor_ms * 1e3, 2), "ours_us": round(ours_ms * 1e3, 2),
            "ours_speedup": round(vendor_ms / ours_ms, 3)}


def sampled_parity(case, y64, npts=2000, seed=0):
    """max|err|/max|ref| over sampled outputs plus the first and last rows."""
    import oracle

    rng = np.random.default_rng(seed)
    mi = np.concatenate([rng.integers(0, case.M, npts), np.repeat([0, case.M - 1], case.N)])
    ni = np.concatenate([rng.integers(0, case.N, npts), np.tile(np.arange(case.N), 2)])
    ref = oracle.linear_points(case.X, case.W, case.b, dtype=case.in_dtype, layout=case.layout, gelu=case.gelu,
                               mi=mi, ni=ni)
    return float(np.max(np.abs(y64[mi, ni] - ref)) / np.max(np.abs(ref)))


def cpu_baseline(budget_s: float = 6.0):
    """The oracle (plain C, fp64 accumulation, OpenMP over output rows) timed on this host's cores.

    Every workload: the whole output on all cores for the small ones (the
    128x768x768 linear, the narrow 16x4096x4096 linear, the 128-row GPT-2
    layer) together with a single-thread run of the whole output; for the
    square 4096^3 GEMM and the M=8192 stack, a row sample on all cores and a
    64-row slice on one thread, scaled to the whole workload and labelled
    extrapolated.  The top-level value is the square fp32 all-core rate, the
    workload the headline measures.
    """
    import oracle
    from dense_gemm_transformer_amd import inputs

    cores = oracle.max_threads()  # before any single-thread call changes the OpenMP default

    def timed(case, rows, threads):
        t0 = time.perf_counter()
        oracle.linear_case(case, threads=threads, rows=rows)
        return time.perf_counter() - t0

    def full(cases):
        flops = sum(c.flops for c in cases)
        t_all = sum(timed(c, None, cores) for c in cases)
        t_one = sum(timed(c, None, 1) for c in cases)
        return {"flops": flops, "all_cores_s": round(t_all, 4), "single_thread_s": round(t_one, 4),
                "all_cores_GFLOP/s": round(flops / t_all / 1e9, 2), "single_thread_GFLOP/s": round(flops / t_one / 1e9, 3),
                "kind": "whole output"}

    def sampled(cases, repeat: int, budget: float):
        """Row sample per GEMM on all cores (about ``budget`` s in total) and a 64-row slice on one thread."""
        flops = repeat * sum(c.flops for c in cases)
        t_all = t_one = 0.0
        rows_all = []
        for c in cases:
            probe = min(c.M, 2 * cores)
            per_row = max(timed(c, (0, probe), cores), 1e-4) / probe
            rows = int(min(c.M, max(probe, budget / len(cases) / per_row)))
            t = timed(c, (0, rows), cores)
            t_all += t * c.M / rows * repeat
            rows_all.append(rows)
            one = min(64, c.M)
            t_one += timed(c, (0, one), 1) * c.M / one * repeat
        return {"flops": flops, "all_cores_s": round(t_all, 3), "single_thread_s": round(t_one, 3),
                "all_cores_GFLOP/s": round(flops / t_all / 1e9, 2), "single_thread_GFLOP/s": round(flops / t_one / 1e9, 3),
                "kind": f"extrapolated: all cores from rows {rows_all} of each GEMM, one thread from 64 rows"
                        + (f", times {repeat} layers" if repeat > 1 else "")}

    per = {}
    per["linear_128x768x768_f32"] = full([inputs.workload_fp32_linear_128x768()])
    per["narrow_16x4096x4096_f16"] = full([inputs.workload_fp16_narrow()])
    per["gpt2_layer_m128_f32"] = full(inputs.workload_gpt2_layer(M=128, dtype="f32"))
    sq = inputs.workload_square(dtype="f32")
    per["square_4096_f32"] = sampled([sq], 1, budget_s)
    per["square_4096_bf16"] = sampled([inputs.workload_square(dtype="bf16")], 1, budget_s / 3)
    for dt in ("f32", "bf16"):
        layer0 = inputs.workload_gpt2_layer(5, 8192, dt, 0)
        per[f"gpt2_stack_m8192_{dt}"] = sampled(layer0, 12, budget_s / 3)
    head = per["square_4096_f32"]
    return {"value": round(head["flops"] / head["all_cores_s"] / 1e12, 5), "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": f"square fp32 4096^3 on {cores} threads, {head['kind']} ({head['all_cores_s']} s for the "
                      "whole output); fp64 accumulation, OpenMP over rows",
            "affinity_cpus": len(os.sched_getaffinity(0)),
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
            "per_workload": per}


def clock_adjusted(ceilings, achieved: float, peak: float, dt: str) -> dict:
    """The datasheet peak scaled to the core clock measured under the MFMA probe (the datasheet
    figure assumes 2400 MHz), and the achieved fraction of it; empty without the probe."""
    if not ceilings:
        return {}
    mhz = ceilings.get(f"sclk_MHz_under_mfma_{dt}")
    if not mhz:
        return {}
    adj = peak * mhz / PEAK_SCLK_MHZ
    return {"sclk_MHz_measured": mhz, "peak_clock_adjusted": round(adj, 2),
            "frac_clock_adjusted": round(achieved / adj, 4)}


def dev_tensor(torch, a, dt, dev):
    """Host storage array (bf16 as raw uint16 bits) -> device tensor."""
    if dt == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def host_f64(torch, t):
    from dense_gemm_transformer_amd import inputs

    t = t.cpu()
    if t.dtype == torch.bfloat16:
        return inputs.widen(t.view(torch.int16).numpy().view(np.uint16), "bf16")
    return t.numpy().astype(np.float64)


def median_span_ms(torch, fn, reps: int, stream) -> float:
    """Median over ``reps`` of the HIP-event span of one call of ``fn()`` on ``stream``."""
    spans = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        b.synchronize()
        spans.append(a.elapsed_time(b))
    return float(np.median(spans))


def graph_span_ms(torch, launch, reps: int, outputs):
    """Capture ``launch(stream_handle)`` in a HIP graph on a side stream; median event span of one replay.

    The replayed outputs are compared bitwise with an eager run first (the
    kernels are deterministic, so a replay must reproduce them exactly).
    """
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())  # the buffers were written on the current stream
    with torch.cuda.stream(side):
        launch(side.cuda_stream)
    side.synchronize()
    want = [o.clone() for o in outputs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        launch(side.cuda_stream)
    for o in outputs:
        o.zero_()
    graph.replay()
    torch.cuda.synchronize()
    same = all(torch.equal(o, w) for o, w in zip(outputs, want))
    for _ in range(3):
        graph.replay()
    ms = median_span_ms(torch, graph.replay, reps, torch.cuda.current_stream())
    del graph
    return ms, same


def bench_ceilings(torch, dev, stream, cold_bufs):
    """Achievable ceilings beside the datasheet peaks: launch floor, plain read, MFMA issue rate."""
    import ctypes

    lib = ctypes.CDLL(os.path.join(ROOT, "dense_gemm_transformer_amd", "libtlgceil.so"))
    vp, s = ctypes.c_void_p, ctypes.c_void_p(stream.cuda_stream)
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    sink = torch.zeros(512, dtype=torch.float32, device=dev)

    def ok(rc):
        if rc != 0:
            raise RuntimeError(f"ceiling probe failed with status {rc}")

    empty_ms = time_launches(lambda i: ok(lib.tlg_ceil_empty(256, vp(flag.data_ptr()), s)), 2000, stream)
    nbytes = cold_bufs[0].numel() * cold_bufs[0].element_size()

    def read(buf):
        ok(lib.tlg_ceil_read(vp(buf.data_ptr()), ctypes.c_size_t(nbytes), vp(sink.data_ptr()), s))

    ramp(lambda i: read(cold_bufs[i % len(cold_bufs)]), stream)
    cold_ms = time_launches(lambda i: read(cold_bufs[i % len(cold_bufs)]), 2000, stream)
    warm_ms = time_launches(lambda i: read(cold_bufs[0]), 2000, stream)
    # on-chip read rate: 256 workgroups re-reading their own 96 KiB blocks of 24 MiB (L2-resident)
    l2buf = torch.zeros(24 << 20, dtype=torch.uint8, device=dev)
    l2_reps = 256
    l2_call = lambda i: ok(lib.tlg_ceil_read_l2(vp(l2buf.data_ptr()), l2_reps, vp(sink.data_ptr()), s))
    ramp(l2_call, stream)
    l2_ms = time_launches(l2_call, 20, stream)
    l2_bytes = (24 << 20) * l2_reps
    del l2buf
    mfma, clock_mhz = {}, {}
    stamps = torch.zeros(4 * 256, dtype=torch.int64, device=dev)
    khz = ctypes.c_int(0)
    ok(lib.tlg_ceil_wall_clock_khz(ctypes.byref(khz)))
    for name, bf16, iters, flop in (("f32", 0, 2000, 4096), ("bf16", 1, 4000, 32768)):
        call = lambda i: ok(lib.tlg_ceil_mfma_clock(bf16, 256, iters, vp(sink.data_ptr()), vp(stamps.data_ptr()), s))
        ramp(call, stream)
        ms = time_launches(call, 10, stream)
        mfma[name] = 256 * 4 * iters * 16 * flop / (ms * 1e-3) / 1e12
        st = stamps.view(256, 4).cpu().numpy().astype(np.float64)  # the last launch's counters
        clock_mhz[name] = float(np.median((st[:, 1] - st[:, 0]) / (st[:, 3] - st[:, 2]))) * khz.value / 1e3
    return {"empty_kernel_event_us": round(empty_ms * 1e3, 3),
            "read_cold_us": round(cold_ms * 1e3, 3), "read_cold_GB/s": round(nbytes / (cold_ms * 1e-3) / 1e9, 1),
            "read_warm_us": round(warm_ms * 1e3, 3), "read_bytes": nbytes,
            "read_l2_GB/s": round(l2_bytes / (l2_ms * 1e-3) / 1e9, 1), "read_l2_bytes_per_launch": l2_bytes,
            "mfma_f32_TFLOP/s": round(mfma["f32"], 1), "mfma_bf16_TFLOP/s": round(mfma["bf16"], 1),
            "sclk_MHz_under_mfma_f32": round(clock_mhz["f32"], 1),
            "sclk_MHz_under_mfma_bf16": round(clock_mhz["bf16"], 1),
            "method": "HIP events over back-to-back launches of the probes in libtlgceil.so: empty kernel "
                      "(256 workgroups), plain read of 32 MiB (256 workgroups x 8 waves x 16 loads of 16 B, "
                      f"cold = rotating {len(cold_bufs)} buffers), on-chip read (256 workgroups re-reading their "
                      f"own 96 KiB blocks of 24 MiB {l2_reps} times, each block in flight at once), "
                      "16 independent 32x32 MFMA chains per wave "
                      "on all CUs; sclk = median over workgroups of shader-clock ticks / constant-rate ticks "
                      "(s_memtime / s_memrealtime) across the MFMA loop, times the constant rate"}



def linear_floor_us(c) -> float:
    """Roofline floor of an fp32 linear with bias: max(flops / MFMA peak, bytes / HBM peak), bytes = X, W, bias
    and Y once each."""
    nbytes = 4 * (c.M * c.K + c.N * c.K + c.N + c.M * c.N)
    return max(c.flops / (PEAK_F32_TFLOPS * 1e12), nbytes / (PEAK_HBM_GBS * 1e9)) * 1e6

def bench_c1(torch, dev, stream, no_parity: bool):
    """fp32 linear 128x768x768 + bias: warm (one W) and cold (128 rotated copies of W, 302 MB)."""
    import oracle
    from dense_gemm_transformer_amd import inputs, tlgemm

    c = inputs.workload_fp32_linear_128x768()
    X, W0, b = (dev_tensor(torch, a, "f32", dev) for a in (c.X, c.W, c.b))
    Y = torch.empty((c.M, c.N), dtype=torch.float32, device=dev)
    plan = tlgemm.Plan.create(c.M, c.N, c.K, "f32", "f32", "NK", True, False)
    ws_bytes = plan.workspace_size
    ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    copies = [W0] + [W0.clone() for _ in range(127)]
    run = lambda w: plan.run_ptrs(X.data_ptr(), w.data_ptr(), b.data_ptr(), Y.data_ptr(),
                                  ws.data_ptr() if ws_bytes else 0, ws_bytes, stream.cuda_stream)
    run(W0)
    torch.cuda.synchronize()
    err = None
    if not no_parity:
        ref = oracle.linear_case(c)
        err = float(np.max(np.abs(host_f64(torch, Y) - ref)) / np.max(np.abs(ref)))
    ramp(lambda i: run(copies[i % len(copies)]), stream)
    cold = time_launches(lambda i: run(copies[i % len(copies)]), 1024, stream)
    warm = time_launches(lambda i: run(W0), 1024, stream)
    # the same launches replayed from HIP graphs: no host work between them
    pX, pb, pY, pw = X.data_ptr(), b.data_ptr(), Y.data_ptr(), ws.data_ptr() if ws_bytes else 0
    g_launch = lambda sh, ws_: [plan.run_ptrs(pX, w.data_ptr(), pb, pY, pw, ws_bytes, sh) for w in ws_]
    g_warm, _ = graph_span_ms(torch, lambda sh: g_launch(sh, [W0] * 32), 20, [Y])
    g_cold, _ = graph_span_ms(torch, lambda sh: g_launch(sh, copies), 20, [Y])
    return {"workload": "fp32 linear Y=X.W^T+b, M=128, K=768, N=768, W out x in, N(0,1)/N(0,0.02)",
            "warm_us": round(warm * 1e3, 3), "cold_us": round(cold * 1e3, 3),
            "warm_graph_us": round(g_warm / 32 * 1e3, 3), "cold_graph_us": round(g_cold / len(copies) * 1e3, 3),
            "TFLOP/s_warm": round(c.flops / (warm * 1e-3) / 1e12, 2),
            "floor_us": round(linear_floor_us(c), 3),
            "frac_of_floor_warm_graph": round(linear_floor_us(c) / (g_warm / 32 * 1e3), 4),
            "parity_err": err, "parity_pass": None if err is None else err <= 1e-5, "plan": plan.describe(),
            "timing": "HIP events over back-to-back launches (includes launch gaps); *_graph_us: median replay "
                      "of a HIP graph of 32 (warm) or 128 (cold, one per weight copy) launches, per launch"}


def bench_c3(torch, dev, stream, no_parity: bool, copies: int = 12):
    """GPT-2-small layer at M=128, fp32: each linear warm, and the four as a layer, warm and cold."""
    import oracle
    from dense_gemm_transformer_amd import inputs, tlgemm

    cases = inputs.workload_gpt2_layer(M=128, dtype="f32")
    gemms = []
    for c in cases:
        X, W, b = (dev_tensor(torch, a, "f32", dev) for a in (c.X, c.W, c.b))
        plan = tlgemm.Plan.create(c.M, c.N, c.K, "f32", "f32", "NK", True, c.gelu)
        ws_bytes = plan.workspace_size
        gemms.append({"case": c, "X": X, "b": b, "Ws": [W] + [W.clone() for _ in range(copies - 1)],
                      "Y": torch.empty((c.M, c.N), dtype=torch.float32, device=dev), "plan": plan,
                      "ws": torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device=dev), "ws_bytes": ws_bytes})

    def run(g, w, sh=None):
        g["plan"].run_ptrs(g["X"].data_ptr(), w.data_ptr(), g["b"].data_ptr(), g["Y"].data_ptr(),
                           g["ws"].data_ptr() if g["ws_bytes"] else 0, g["ws_bytes"],
                           stream.cuda_stream if sh is None else sh)

    out = {"workload": "GPT-2-small layer linears at M=128, fp32, bias on all, tanh-GELU on fc; "
                       f"cold = {copies} rotated weight sets ({copies} x 28.3 MB)", "gemms": {}}
    for g in gemms:
        run(g, g["Ws"][0])
    torch.cuda.synchronize()
    for g in gemms:
        c = g["case"]
        ramp(lambda i: run(g, g["Ws"][0]), stream)
        err = None
        if not no_parity:
            ref = oracle.linear_case(c)
            err = float(np.max(np.abs(host_f64(torch, g["Y"]) - ref)) / np.max(np.abs(ref)))
        warm = time_launches(lambda i: run(g, g["Ws"][0]), 512, stream)
        out["gemms"][c.name] = {"warm_us": round(warm * 1e3, 3),
                                "TFLOP/s_warm": round(c.flops / (warm * 1e-3) / 1e12, 2),
                                "floor_us": round(linear_floor_us(c), 3),
                                "frac_of_floor_warm": round(linear_floor_us(c) / (warm * 1e3), 4),
                                "parity_err": err, "plan": g["plan"].describe()}

    def layer(l):
        for g in gemms:
            run(g, g["Ws"][l % copies])

    ramp(layer, stream)
    warm = time_launches(lambda i: layer(0), 256, stream)
    cold = time_launches(lambda i: layer(i), 256, stream)
    flops = sum(g["case"].flops for g in gemms)
    single_ms = median_span_ms(torch, lambda: layer(0), 200, stream)
    graph_ms, graph_same = graph_span_ms(torch, lambda sh: [run(g, g["Ws"][0], sh) for g in gemms], 200,
                                         [g["Y"] for g in gemms])
    out.update({"layer_single_eager_us": round(single_ms * 1e3, 3), "layer_single_graph_us": round(graph_ms * 1e3, 3),
                "layer_graph_bitwise_equal": graph_same})
    out.update({"layer_warm_us": round(warm * 1e3, 3), "layer_cold_us": round(cold * 1e3, 3),
                "layer_TFLOP/s_cold": round(flops / (cold * 1e-3) / 1e12, 2),
                "timing": "HIP events over back-to-back layers of four launches (includes launch gaps); "
                          "layer_single_eager_us / layer_single_graph_us: median event span of one isolated layer, "
                          "launched eagerly or replayed from a HIP graph of its four launches (warm weights)"})
    out["parity_pass"] = None if no_parity else all(v["parity_err"] <= 1e-5 for v in out["gemms"].values())
    return out


def bench_c5(torch, dev, stream, dtype: str, no_parity: bool, layers: int = 12, reps: int = 20,
             vendor: bool = True):
    """Batched GPT-2-small stack at M=8192: one pass = 12 layers x 4 linears, 48 launches on one stream."""
    from dense_gemm_transformer_amd import inputs, tlgemm

    M, w = 8192, 5
    peak = PEAK_F32_TFLOPS if dtype == "f32" else PEAK_BF16_TFLOPS
    xs, plans, ys, wb = [], [], [], []
    for g, (name, N, K, gelu) in enumerate(inputs.GPT2_LINEARS):
        x0 = dev_tensor(torch, inputs.gpt2_activation(w, 0, g, M, dtype), dtype, dev)
        # later layers read row-rotated copies of layer 0's activations: distinct memory, same values
        xs.append([x0] + [torch.roll(x0, shifts=97 * l, dims=0).contiguous() for l in range(1, layers)])
        plans.append(tlgemm.Plan.create(M, N, K, dtype, dtype, "NK", True, gelu))
        ys.append(torch.empty((M, N), dtype=tlgemm.torch_dtype(dtype), device=dev))
    for l in range(layers):
        row = []
        for g in range(4):
            W, b = inputs.gpt2_weights(w, l, g, dtype)
            row.append((dev_tensor(torch, W, dtype, dev), dev_tensor(torch, b, dtype, dev)))
        wb.append(row)
    wss = [torch.zeros(max(p.workspace_size, 1), dtype=torch.uint8, device=dev) for p in plans]

    def one_pass(sh=None):
        for l in range(layers):
            for g in range(4):
                p, (W, b) = plans[g], wb[l][g]
                p.run_ptrs(xs[g][l].data_ptr(), W.data_ptr(), b.data_ptr(), ys[g].data_ptr(),
                           wss[g].data_ptr() if p.workspace_size else 0, p.workspace_size,
                           stream.cuda_stream if sh is None else sh)

    errs = {}
    if not no_parity:  # layer 0 of each linear, sampled against the oracle
        for g, (name, N, K, gelu) in enumerate(inputs.GPT2_LINEARS):
            p, (W, b) = plans[g], wb[0][g]
            p.run_ptrs(xs[g][0].data_ptr(), W.data_ptr(), b.data_ptr(), ys[g].data_ptr(),
                       wss[g].data_ptr() if p.workspace_size else 0, p.workspace_size, stream.cuda_stream)
            torch.cuda.synchronize()
            Wh, bh = inputs.gpt2_weights(w, 0, g, dtype)
            case = inputs.LinearCase(name, M, N, K, dtype, dtype, "NK", True, gelu,
                                     inputs.gpt2_activation(w, 0, g, M, dtype), Wh, bh)
            errs[name] = sampled_parity(case, host_f64(torch, ys[g]), npts=1000)
    ramp(lambda i: one_pass(), stream)
    ms = median_span_ms(torch, one_pass, reps, stream)
    graph_ms, graph_same = graph_span_ms(torch, one_pass, reps, ys)
    flops = layers * sum(2 * M * N * K for _, N, K, _ in inputs.GPT2_LINEARS)
    tol = 1e-5 if dtype == "f32" else 1e-2
    vend = None
    if vendor:  # the same 48 products through the vendor library (GELU a kernel of its own), same inputs

        def vendor_pass():
            for l in range(layers):
                for g in range(4):
                    W, b = wb[l][g]
                    y = torch.nn.functional.linear(xs[g][l], W, b)
                    if inputs.GPT2_LINEARS[g][3]:
                        torch.nn.functional.gelu(y, approximate="tanh")

        tf32 = torch.backends.cuda.matmul.allow_tf32
        torch.backends.cuda.matmul.allow_tf32 = False
        ramp(lambda i: vendor_pass(), stream)
        vend = vendor_entry("F.linear(x, W, b) per product, then F.gelu(tanh) on fc; TF32 off",
                            median_span_ms(torch, vendor_pass, reps, stream), ms)
        torch.backends.cuda.matmul.allow_tf32 = tf32
    return {"workload": f"GPT-2-small stack, M=8192 (64 x 128 tokens), {layers} layers x "
                        "{qkv, attn-out, fc+GELU, proj}, bias on all, " + dtype + " in and out",
            "pass_ms": round(ms, 4), "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 2),
            "frac_mfma_peak": round(flops / (ms * 1e-3) / 1e12 / peak, 4),
            "tokens_per_s": round(M / (ms * 1e-3), 1), "flops_per_pass": flops,
            "pass_ms_graph": round(graph_ms, 4), "TFLOP/s_graph": round(flops / (graph_ms * 1e-3) / 1e12, 2),
            "graph_bitwise_equal": graph_same,
            "parity_err_layer0": errs or None,
            "parity_pass": None if not errs else all(e <= tol for e in errs.values()),
            "plans": [p.describe() for p in plans],
            "vendor_library": vend,
            "timing": f"median over {reps} passes of the HIP-event span of one pass (48 launches, one stream); "
                      "12 distinct weight sets, activations of later layers are row-rotated copies of layer 0's; "
                      "pass_ms_graph: the same 48 launches captured once in a HIP graph, median replay span"}


def bench_backward(torch, dev, stream, dtype: str, no_parity: bool, reps: int = 20):
    """Backward GEMMs of the four GPT-2-small linears at 8192 tokens: dX = dY·W (weight read [K][N]) and
    dW = dYᵀ·X accumulated onto an existing gradient (first operand stored transposed, residual flag)."""
    from dense_gemm_transformer_amd import inputs, tlgemm

    T = 8192
    peak = PEAK_F32_TFLOPS if dtype == "f32" else PEAK_BF16_TFLOPS
    cases = inputs.workload_gpt2_backward(T=T, dtype=dtype)
    nl = len(inputs.GPT2_LINEARS)
    jobs = []
    for g, (name, N, K, _) in enumerate(inputs.GPT2_LINEARS):
        cx, cw = cases[g], cases[nl + g]
        d = {"W": dev_tensor(torch, cx.W, dtype, dev), "dY": dev_tensor(torch, cx.X, dtype, dev),
             "X": dev_tensor(torch, cw.W, dtype, dev), "G": dev_tensor(torch, cw.R, dtype, dev)}
        dx = tlgemm.Plan.create(cx.M, cx.N, cx.K, dtype, dtype, cx.layout)
        dw = tlgemm.Plan.create(cw.M, cw.N, cw.K, dtype, dtype, cw.layout, residual=True)
        outs = {"dX": torch.empty((T, K), dtype=tlgemm.torch_dtype(dtype), device=dev), "dW": d["G"].clone()}
        wss = [torch.zeros(max(p.workspace_size, 1), dtype=torch.uint8, device=dev) for p in (dx, dw)]
        jobs.append((name, dx, dw, d, outs, wss, (cx.X, cx.W, cw.W, cw.R)))

    def one_pass():
        for name, dx, dw, d, outs, wss, _ in jobs:
            dx.run_ptrs(d["dY"].data_ptr(), d["W"].data_ptr(), 0, outs["dX"].data_ptr(),
                        wss[0].data_ptr() if dx.workspace_size else 0, dx.workspace_size, stream.cuda_stream)
            dw.run_ptrs(d["dY"].data_ptr(), d["X"].data_ptr(), 0, outs["dW"].data_ptr(),
                        wss[1].data_ptr() if dw.workspace_size else 0, dw.workspace_size, stream.cuda_stream)

    errs = {}
    if not no_parity:  # one pass from the initial gradients, sampled against the oracle
        import oracle

        one_pass()
        torch.cuda.synchronize()
        rng = np.random.default_rng(0)
        tol = 1e-5 if dtype == "f32" else 1e-2
        for name, dx, dw, d, outs, wss, (dY, W, X, G) in jobs:
            for key, out, A, B, lay, R in (("dX", outs["dX"], dY, W, "KN", None),
                                           ("dW", outs["dW"], dY, X, "AT_KN", G)):
                M, N = out.shape
                mi, ni = rng.integers(0, M, 1000), rng.integers(0, N, 1000)
                ref = oracle.linear_points(A, B, None, dtype=dtype, layout=lay, mi=mi, ni=ni, residual=R,
                                           out_dtype=dtype)
                y = host_f64(torch, out)
                errs[f"{name}.{key}"] = float(np.max(np.abs(y[mi, ni] - ref)) / np.max(np.abs(ref)))
        for name, dx, dw, d, outs, wss, _ in jobs:  # back to the initial gradients for timing
            outs["dW"].copy_(d["G"])
    ramp(lambda i: one_pass(), stream)
    ms = median_span_ms(torch, one_pass, reps, stream)
    flops = sum(2 * 2 * T * N * K for _, N, K, _ in inputs.GPT2_LINEARS)
    return {"workload": f"GPT-2-small backward GEMMs at {T} tokens, one layer: dX = dY.W ([K][N] weight) and "
                        f"dW += dY^T.X (first operand stored transposed, residual accumulate) for qkv, attn-out, "
                        f"fc, proj; {dtype}",
            "pass_ms": round(ms, 4), "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 2),
            "frac_mfma_peak": round(flops / (ms * 1e-3) / 1e12 / peak, 4), "flops_per_pass": flops,
            "parity_err": errs or None,
            "parity_pass": None if not errs else all(e <= (1e-5 if dtype == "f32" else 1e-2) for e in errs.values()),
            "plans": [p.describe() for job in jobs for p in (job[1], job[2])],
            "timing": f"median over {reps} passes of the HIP-event span of one pass (8 launches, one stream); "
                      "dW accumulates onto itself from pass to pass"}


def bench_layer_ops(torch, dev, stream, dtype: str, no_parity: bool, reps: int = 50):
    """LayerNorm over the GPT-2-small stack's 8192 x 768 activations and fused causal attention over its
    64 x 128 x 12-head qkv projection: HBM-bound, so bytes per launch against 8 TB/s."""
    from dense_gemm_transformer_amd import inputs, layer

    es = 4 if dtype == "f32" else 2
    X, g, b = inputs.workload_gpt2_layernorm(dtype=dtype)
    rows, C = X.shape
    dX, dg, db = (dev_tensor(torch, a, dtype, dev) for a in (X, g, b))
    dY = torch.empty_like(dX)
    pX, pg, pb, pY = dX.data_ptr(), dg.data_ptr(), db.data_ptr(), dY.data_ptr()
    ln = lambda sh: layer.tlg_layernorm(pX, pg, pb, pY, 0, 0, rows, C, 1e-5, dtype, sh)
    B, T, NH, HS = 64, 128, 12, 64
    qkv = inputs.workload_gpt2_attention(B=B, T=T, n_head=NH, head_size=HS, dtype=dtype)
    dqkv = dev_tensor(torch, qkv, dtype, dev)
    dout = torch.empty((B, T, NH * HS), dtype=dqkv.dtype, device=dev)
    pq, po = dqkv.data_ptr(), dout.data_ptr()
    att = lambda sh: layer.tlg_attention(pq, po, 0, B, T, NH, HS, dtype, True, sh)
    res = {}
    per_graph = 32  # launches captured in one graph
    for name, fn, out, nbytes, flops in (
            ("layernorm_8192x768", ln, dY, rows * C * 2 * es + 2 * C * es, None),
            ("attention_b64_t128_h12", att, dout, B * T * 4 * NH * HS * es, 4 * B * NH * HS * T * (T + 1) // 2)):
        fn(stream.cuda_stream)
        torch.cuda.synchronize()
        ramp(lambda i: fn(stream.cuda_stream), stream)
        us_eager = time_launches(lambda i: fn(stream.cuda_stream), reps, stream) * 1e3
        # The host issues a launch through the Python binding in about as long as these kernels run, so
        # back-to-back eager launches can measure the host: the primary figure replays per_graph launches
        # captured in one HIP graph (no host work between them), per launch.
        g_ms, g_same = graph_span_ms(torch, lambda sh: [fn(sh) for _ in range(per_graph)], reps, [out])
        us = g_ms / per_graph * 1e3
        r = {"us": round(us, 3), "us_eager": round(us_eager, 3), "graph_bitwise_equal": g_same,
             "GB/s": round(nbytes / us / 1e3, 1),
             "roofline": {"bound": "hbm", "achieved": round(nbytes / us / 1e3, 1), "peak": PEAK_HBM_GBS,
                          "unit": "GB/s", "frac": round(nbytes / us / 1e3 / PEAK_HBM_GBS, 4),
                          "algorithmic_bytes_per_launch": nbytes}}
        if flops:
            r["TFLOP/s"] = round(flops / us / 1e6, 2)
        res[name] = r
    if not no_parity:
        import oracle

        ref, _, _ = oracle.layernorm(X, g, b, dtype=dtype)
        res["layernorm_8192x768"]["parity_err"] = oracle.normalized_error(host_f64(torch, dY), ref)
        ref, _ = oracle.attention(qkv[:4], NH, dtype=dtype)  # the first 4 sequences
        res["attention_b64_t128_h12"]["parity_err"] = oracle.normalized_error(host_f64(torch, dout)[:4], ref)
        tol = 1e-5 if dtype == "f32" else 1e-2
        for k in res:
            res[k]["parity_pass"] = res[k]["parity_err"] <= tol
    res["timing"] = (f"us: median over {reps} replays of a HIP graph of {per_graph} back-to-back launches, per "
                     f"launch; us_eager: HIP events over {reps} launches from Python on one stream (host-bound "
                     "where the binding's call takes longer than the kernel)")
    res["workload"] = (f"GPT-2-small layer ops, {dtype}: LayerNorm of X [{rows}][{C}] (gamma, beta), fused causal "
                       f"attention over qkv [{B}][{T}][{3 * NH * HS}] ({NH} heads of {HS}), no lse")
    return res


def bench_gpt2_forward(torch, dev, stream, dtype: str, no_parity: bool, layers: int = 12, reps: int = 10):
    """GPT-2-small forward through ``layers`` transformer blocks at 64 x 128 tokens: per block two LayerNorms,
    the qkv projection, fused causal attention, the attention output projection and proj with the residual
    fused, fc with GELU (7 launches; embeddings, final LayerNorm and logits excluded)."""
    from dense_gemm_transformer_amd import block, inputs

    B, T, C, NH = 64, 128, 768, 12
    shape = block.BlockShape(B, T, C, NH, dtype)
    blocks = []
    params0 = None
    for li in range(layers):
        P = inputs.gpt2_block_params(10, li, C, dtype)
        if li == 0:
            params0 = P
        blocks.append(block.GPT2Block(shape, {k: dev_tensor(torch, v, dtype, dev) for k, v in P.items()}))
    x0 = inputs.normal(inputs.seed_for(10, 0, 1), (B * T, C), 1.0, dtype)
    x = dev_tensor(torch, x0, dtype, dev)
    res = {}
    if not no_parity:  # the first block on a fresh input, its first two sequences against the oracle stages
        import oracle

        blocks[0].forward(x, stream.cuda_stream)
        torch.cuda.synchronize()
        st = lambda a: inputs.store(a, dtype)
        rows = 2 * T
        xs = x0[:rows]
        Pp = params0
        h, _, _ = oracle.layernorm(xs, Pp["ln1_g"], Pp["ln1_b"], dtype=dtype)
        qkv = oracle.linear(st(h), Pp["w_qkv"], Pp["b_qkv"], dtype=dtype)
        att, _ = oracle.attention(st(qkv).reshape(2, T, -1), NH, dtype=dtype)
        x1 = oracle.linear(st(att.reshape(rows, -1)), Pp["w_attn"], Pp["b_attn"], dtype=dtype, residual=xs)
        h2, _, _ = oracle.layernorm(st(x1), Pp["ln2_g"], Pp["ln2_b"], dtype=dtype)
        f = oracle.linear(st(h2), Pp["w_fc"], Pp["b_fc"], dtype=dtype, gelu=True)
        ref = oracle.linear(st(f), Pp["w_proj"], Pp["b_proj"], dtype=dtype, residual=st(x1))
        res["parity_err_block0"] = oracle.normalized_error(host_f64(torch, x)[:rows], ref)
        res["parity_pass"] = res["parity_err_block0"] <= (1e-5 if dtype == "f32" else 1e-2)
        x.copy_(dev_tensor(torch, x0, dtype, dev))

    def one_pass():
        for blk in blocks:
            blk.forward(x, stream.cuda_stream)

    ramp(lambda i: one_pass(), stream)
    ms = median_span_ms(torch, one_pass, reps, stream)
    # the same pass captured once in a HIP graph, starting from a device copy of the input
    xin = dev_tensor(torch, x0, dtype, dev)

    def graph_pass(s):  # called with the capturing stream current
        x.copy_(xin)
        for blk in blocks:
            blk.forward(x, s)

    ms_graph, same = graph_span_ms(torch, graph_pass, reps, [x])
    flops = layers * shape.flops()
    peak = PEAK_F32_TFLOPS if dtype == "f32" else PEAK_BF16_TFLOPS
    res.update({"pass_ms_graph": round(ms_graph, 4), "graph_bitwise_equal": same})
    res.update({"workload": f"GPT-2-small forward through {layers} blocks, {B} x {T} tokens, {dtype}: per block "
                            "LayerNorm, qkv, fused causal attention, attn-out (+residual), LayerNorm, fc+GELU, "
                            "proj (+residual); no embeddings, final LayerNorm or logits",
                "pass_ms": round(ms, 4), "tokens_per_s": round(B * T / (ms * 1e-3), 1),
                "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 2),
                "frac_mfma_peak": round(flops / (ms * 1e-3) / 1e12 / peak, 4), "flops_per_pass": flops,
                "launches_per_pass": 7 * layers,
                "timing": f"median over {reps} passes of the HIP-event span of one pass on one stream; pass_ms_graph: "
                          "the pass (plus a copy of the input into place) captured once in a HIP graph, median "
                          "replay span, its output bitwise equal to the eager pass"})
    return res


def rocprof_summary(outdir: str, segments: list[str]) -> str:
    """Markdown summary of a ``rocprofv3 --kernel-trace --stats --output-format csv`` run under ``outdir``.

    One row per (kernel, launch grid in workgroups): launches, median, p10,
    p90 and minimum duration, so that kernels of one template with different
    tiles or grids are never pooled.  The library's kernels and the ceiling
    probes only: torch's and the HIP runtime's own kernels are left out.  ``segments`` entries ``NAME@GRID=n1,n2,...``
    split that row's launches, in dispatch order, into consecutive runs of
    n1, n2, ... launches (for example the parity call, the clock ramp, the
    cold launches and the warm launches of one kernel), each summarised on its
    own; one ``*`` stands for however many launches the other runs leave (the
    ramp's count depends on the clock).
    """
    import csv

    traces = sorted(glob.glob(os.path.join(outdir, "**", "*kernel_trace.csv"), recursive=True))
    stats = sorted(glob.glob(os.path.join(outdir, "**", "*kernel_stats.csv"), recursive=True))
    if not traces:
        raise SystemExit(f"no kernel_trace.csv under {outdir}")
    groups: dict = {}
    for path in traces:
        with open(path, newline="") as f:
            for row in csv.DictReader(f):
                wg = [int(row[f"Workgroup_Size_{a}"]) for a in "XYZ"]
                grid = [int(row[f"Grid_Size_{a}"]) // max(w, 1) for a, w in zip("XYZ", wg)]
                key = (row["Kernel_Name"], "x".join(map(str, grid)))
                dur = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3
                groups.setdefault(key, []).append((int(row["Dispatch_Id"]), dur))
    def short(name: str) -> str:  # the template arguments identify a kernel; drop its parameter list
        return name[:name.rindex("(")] if name.endswith(")") and "(" in name else name

    def ours(name: str) -> bool:  # the library's kernels and the ceiling probes, not torch's, BLAS's or the runtime's
        return not name.startswith(("void at::", "at::", "__amd_rocclr", "Cijk_", "Custom_Cijk", "rocblas",
                                    "void rocblas", "void hipblaslt"))

    lines = ["| kernel | grid (workgroups) | launches | median µs | p10 µs | p90 µs | min µs |",
             "|---|---|---|---|---|---|---|"]
    for (name, grid), v in sorted(groups.items(), key=lambda kv: -sum(d for _, d in kv[1])):
        if not ours(name):
            continue
        d = np.array([x for _, x in v])
        lines.append(f"| `{short(name)}` | {grid} | {len(d)} | {np.median(d):.2f} | {np.percentile(d, 10):.2f} | "
                     f"{np.percentile(d, 90):.2f} | {d.min():.2f} |")
    out = ["Per launch configuration (kernel begin to end, from the kernel trace):", "", *lines, ""]
    for spec in segments:
        key, counts = spec.rsplit("=", 1)
        name, grid = key.rsplit("@", 1)
        v = sorted(groups.get((name, grid), []))
        parts = counts.split(",")
        if parts.count("*") > 1:
            raise SystemExit(f"{spec}: at most one '*' run")
        fixed = sum(int(c) for c in parts if c != "*")
        sizes = [len(v) - fixed if c == "*" else int(c) for c in parts]  # '*': the launches the others leave
        if sum(sizes) != len(v) or min(sizes) < 0:
            raise SystemExit(f"{name}@{grid}: {len(v)} launches in the trace, segments sum to {sum(sizes)}")
        out += [f"`{short(name)}` at grid {grid}, launches in dispatch order split into runs of {counts}:", "",
                "| run | launches | median µs | p10 µs | p90 µs |", "|---|---|---|---|---|"]
        i = 0
        for k, n in enumerate(sizes):
            d = np.array([x for _, x in v[i:i + n]])
            i += n
            out.append(f"| {k} | {n} | {np.median(d):.2f} | {np.percentile(d, 10):.2f} | {np.percentile(d, 90):.2f} |")
        out.append("")
    for path in stats:
        with open(path, newline="") as f:
            rows = list(csv.DictReader(f))
        out += [f"rocprofv3 `--stats` ({os.path.basename(path)}):", "",
                "| kernel | calls | average µs | min µs | max µs |", "|---|---|---|---|---|"]
        for r in rows:
            if not ours(r["Name"]):
                continue
            out.append(f"| `{short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                       f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
        out.append("")
        # the vendor GEMMs of the bench's context leg, by the macro tile and MFMA tokens their names carry
        vend = [r for r in rows if r["Name"].startswith(("Cijk_", "Custom_Cijk"))]
        if vend:
            out += ["Vendor BLAS kernels in the same run (`--stats`), by the macro-tile and MFMA tokens of their names:",
                    "", "| macro tile, MFMA | calls | average µs |", "|---|---|---|"]
            for r in vend:
                tag = " ".join(t for t in r["Name"].split("_") if t.startswith(("MT", "MI")))
                out.append(f"| {tag} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} |")
            out.append("")
    return "\n".join(out)


def pmc_summary(fetch_dir: str, write_dir: str, kernels: list[str]) -> str:
    """Markdown table of HBM bytes per launch from two ``rocprofv3 --pmc`` runs (FETCH_SIZE, WRITE_SIZE).

    Both counters read KiB per dispatch.  Each is scaled by the factor that
    makes it read the true size of the runtime's device-to-device copies in
    the same run (``__amd_rocclr_copyBuffer`` of one 32 MiB weight copy).
    ``kernels`` entries ``NAME@GRID=ALGORITHMIC_BYTES`` name the rows to report.
    """
    import csv

    def per_kernel(d: str, counter: str):
        out: dict = {}
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path, newline="") as f:
                for row in csv.DictReader(f):
                    if row["Counter_Name"] != counter:
                        continue
                    wg = max(int(row["Workgroup_Size"]), 1)
                    key = (row["Kernel_Name"], f"{int(row['Grid_Size']) // wg}x1x1")
                    out.setdefault(key, []).append(float(row["Counter_Value"]))
        return out

    fetch, write = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")
    copy = [k for k in fetch if k[0].startswith("__amd_rocclr_copyBuffer") and k[1] == "256x1x1"]
    if not copy:
        raise SystemExit("no 32 MiB device copy in the FETCH_SIZE run to calibrate against")
    kib = 32 * 1024.0
    f_scale = kib / float(np.median(fetch[copy[0]]))
    w_scale = kib / float(np.median(write[copy[0]]))
    lines = [f"Calibration: the 32 MiB device copies read FETCH_SIZE {kib / f_scale:.1f} KiB and WRITE_SIZE "
             f"{kib / w_scale:.1f} KiB, so FETCH_SIZE is scaled by {f_scale:.3f} and WRITE_SIZE by {w_scale:.3f}.", "",
             "| kernel | grid | launches | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled bytes per launch | algorithmic bytes | ratio |",
             "|---|---|---|---|---|---|---|---|"]
    for spec in kernels:
        key, alg = spec.rsplit("=", 1)
        name, grid = key.rsplit("@", 1)
        fk = [k for k in fetch if k[0].startswith(name) and k[1] == grid]
        if len(fk) != 1:
            raise SystemExit(f"{name}@{grid}: {len(fk)} matching kernels in the FETCH_SIZE run")
        fv, wv = float(np.median(fetch[fk[0]])), float(np.median(write.get(fk[0], [0.0])))
        tot = fv * 1024 * f_scale + wv * 1024 * w_scale
        shown = fk[0][0][:fk[0][0].rindex("(")] if fk[0][0].endswith(")") else fk[0][0]
        lines.append(f"| `{shown}` | {grid} | {len(fetch[fk[0]])} | {fv:.1f} | {wv:.1f} | {tot:.0f} | {alg} | "
                     f"{tot / float(alg):.2f} |")
    return "\n".join(lines)


def counter_summary(dirs: list[str], kernels: list[str]) -> str:
    """Markdown table of per-dispatch counter medians from ``rocprofv3 --pmc`` runs (any counters).

    ``kernels`` entries ``NAME@GRID`` name the rows.  GRBM_GUI_ACTIVE reads
    the busy cycles of the 8 XCDs summed: over 8 it is the kernel's length in
    core-clock cycles, and over the kernel's median duration in the same run's
    kernel trace, its core clock.  Where the run holds them, derived columns
    follow: that clock; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES over the 1024
    SIMDs times the kernel's cycles; the LDS bank-conflict share =
    SQ_LDS_BANK_CONFLICT over SQ_LDS_IDX_ACTIVE.
    """
    import csv

    vals: dict = {}
    durs: dict = {}
    for d in dirs:
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path, newline="") as f:
                for row in csv.DictReader(f):
                    wg = max(int(row["Workgroup_Size"]), 1)
                    key = (row["Kernel_Name"], f"{int(row['Grid_Size']) // wg}x1x1")
                    vals.setdefault(key, {}).setdefault(row["Counter_Name"], []).append(float(row["Counter_Value"]))
        for path in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True):
            with open(path, newline="") as f:
                for row in csv.DictReader(f):
                    wg = (max(int(row["Workgroup_Size_X"]), 1), max(int(row["Workgroup_Size_Y"]), 1),
                          max(int(row["Workgroup_Size_Z"]), 1))
                    grid = tuple(int(row[f"Grid_Size_{a}"]) // w for a, w in zip("XYZ", wg))
                    if grid[1:] == (1, 1):
                        durs.setdefault((row["Kernel_Name"], f"{grid[0]}x1x1"), []).append(
                            (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) * 1e-9)
    names = sorted({c for v in vals.values() for c in v})
    xcds, simds = 8, 1024
    derived = []
    if "GRBM_GUI_ACTIVE" in names:
        derived.append(("core MHz", lambda m, t: m["GRBM_GUI_ACTIVE"] / xcds / t / 1e6 if t else float("nan")))
    if "SQ_VALU_MFMA_BUSY_CYCLES" in names and "GRBM_GUI_ACTIVE" in names:
        derived.append(("MFMA busy",
                        lambda m, t: m["SQ_VALU_MFMA_BUSY_CYCLES"] / (m["GRBM_GUI_ACTIVE"] / xcds * simds)))
    if "SQ_LDS_BANK_CONFLICT" in names and "SQ_LDS_IDX_ACTIVE" in names:
        derived.append(("LDS conflict share",
                        lambda m, t: m["SQ_LDS_BANK_CONFLICT"] / max(m["SQ_LDS_IDX_ACTIVE"], 1.0)))
    lines = ["| kernel | grid | dispatches | median µs | " + " | ".join(names + [d[0] for d in derived]) + " |",
             "|---|---|---|---|" + "---|" * (len(names) + len(derived))]
    for spec in kernels:
        name, grid = spec.rsplit("@", 1)
        ks = [k for k in vals if k[0].startswith(name) and k[1] == grid]
        if len(ks) != 1:
            raise SystemExit(f"{name}@{grid}: {len(ks)} matching kernels in the counter runs")
        v = vals[ks[0]]
        med = {c: float(np.median(v[c])) for c in v}
        shown = ks[0][0][:ks[0][0].rindex("(")] if ks[0][0].endswith(")") else ks[0][0]
        t = float(np.median(durs[ks[0]])) if ks[0] in durs else 0.0
        cells = [f"{med[c]:.4g}" if c in med else "" for c in names]
        cells += [f"{fn(med, t):.3f}" if all(c in med for c in names) else "" for _, fn in derived]
        lines.append(f"| `{shown}` | {grid} | {max(len(x) for x in v.values())} | {t * 1e6:.2f} | "
                     + " | ".join(cells) + " |")
    return "\n".join(lines)


def main(argv=None) -> int:
    global RAMP_MS
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50, help="timed square-GEMM steps")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--ramp-ms", type=float, default=RAMP_MS,
                    help="untimed back-to-back work before each timed region, in GPU milliseconds (clock ramp)")
    ap.add_argument("--narrow-launches", type=int, default=2000, help="timed cold narrow launches")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--no-vendor", action="store_true",
                    help="skip the vendor-library context (torch.mm / F.linear, i.e. hipBLASLt or rocBLAS)")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the ceiling probes and the 128-row layer and M=8192 stack workloads")
    ap.add_argument("--rocprof-summary", metavar="DIR",
                    help="print a markdown summary of a rocprofv3 kernel-trace run under DIR and exit (no GPU)")
    ap.add_argument("--counter-summary", nargs="+", metavar="DIR",
                    help="print per-dispatch counter medians of rocprofv3 --pmc runs under the DIRs and exit (no GPU)")
    ap.add_argument("--segment", action="append", default=[], metavar="NAME@GRID=n1,n2,...",
                    help="with --rocprof-summary: split one kernel's launches into consecutive runs")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print HBM bytes per launch from FETCH_SIZE / WRITE_SIZE rocprofv3 runs and exit (no GPU)")
    ap.add_argument("--kernel", action="append", default=[], metavar="NAME@GRID=BYTES",
                    help="with --pmc-summary: a kernel row to report, with its algorithmic bytes per launch; "
                         "with --counter-summary: NAME@GRID")
    args = ap.parse_args(argv)
    RAMP_MS = args.ramp_ms

    if args.pmc_summary:
        print(pmc_summary(args.pmc_summary[0], args.pmc_summary[1], args.kernel))
        return 0
    if args.counter_summary:
        print(counter_summary(args.counter_summary, args.kernel))
        return 0
    if args.rocprof_summary:
        print(rocprof_summary(args.rocprof_summary, args.segment))
        return 0

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): this library has no multi-GPU path.",
              file=sys.stderr)
        return 2

    import torch

    from dense_gemm_transformer_amd import inputs, tlgemm

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    clocks_before = read_clocks(torch)

    def to_dev(a, dt):
        if dt == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def to_f64(t):
        t = t.cpu()
        if t.dtype == torch.bfloat16:
            return inputs.widen(t.view(torch.int16).numpy().view(np.uint16), "bf16")
        return t.numpy().astype(np.float64)

    # ---- square fp32 GEMM 4096³ (the step) ----------------------------------------------
    log("square fp32 4096^3: generating inputs")
    sq = inputs.workload_square(dtype="f32")
    A, B = to_dev(sq.X, "f32"), to_dev(sq.W, "f32")
    C = torch.empty((sq.M, sq.N), dtype=torch.float32, device=dev)
    plan = tlgemm.Plan.create(sq.M, sq.N, sq.K, "f32", "f32", "KN")
    run_sq = lambda i: plan.run_ptrs(A.data_ptr(), B.data_ptr(), 0, C.data_ptr(), 0, 0, stream.cuda_stream)
    run_sq(0)
    torch.cuda.synchronize()
    sq_err = None if args.no_parity else sampled_parity(sq, to_f64(C))
    log(f"square fp32: {plan.describe()} parity {sq_err}")
    ramp(run_sq, stream, args.ramp_ms)
    for i in range(args.warmup):
        run_sq(i)
    ms = time_launches(run_sq, args.steps, stream)
    sq_tflops = sq.flops / (ms * 1e-3) / 1e12
    log(f"square fp32: {ms * 1e3:.1f} us/step, {sq_tflops:.1f} TFLOP/s")

    # bf16 inputs, fp32 output (same shape), reported beside
    sqb = inputs.workload_square(dtype="bf16")
    Ab, Bb = to_dev(sqb.X, "bf16"), to_dev(sqb.W, "bf16")
    planb = tlgemm.Plan.create(sqb.M, sqb.N, sqb.K, "bf16", "f32", "KN")
    run_sqb = lambda i: planb.run_ptrs(Ab.data_ptr(), Bb.data_ptr(), 0, C.data_ptr(), 0, 0, stream.cuda_stream)
    run_sqb(0)
    torch.cuda.synchronize()
    sqb_err = None if args.no_parity else sampled_parity(sqb, to_f64(C))
    ramp(run_sqb, stream, args.ramp_ms)
    for i in range(args.warmup):
        run_sqb(i)
    msb = time_launches(run_sqb, args.steps, stream)
    log(f"square bf16: {msb * 1e3:.1f} us, {sqb.flops / (msb * 1e-3) / 1e12:.1f} TFLOP/s, parity {sqb_err}")
    # the same product with bf16 output (the planner's choice for a shape the table does not list)
    Cb = torch.empty((sqb.M, sqb.N), dtype=torch.bfloat16, device=dev)
    planbb = tlgemm.Plan.create(sqb.M, sqb.N, sqb.K, "bf16", "bf16", "KN")
    run_sqbb = lambda i: planbb.run_ptrs(Ab.data_ptr(), Bb.data_ptr(), 0, Cb.data_ptr(), 0, 0, stream.cuda_stream)
    run_sqbb(0)
    torch.cuda.synchronize()
    sqbb_err = None if args.no_parity else sampled_parity(sqb, to_f64(Cb))
    ramp(run_sqbb, stream, args.ramp_ms)
    msbb = time_launches(run_sqbb, args.steps, stream)
    log(f"square bf16 -> bf16: {msbb * 1e3:.1f} us, parity {sqbb_err}")
    # The vendor library (torch.mm: hipBLASLt or rocBLAS) on the same inputs, for context: the same ramp, the
    # same event timing, fp32 arithmetic (TF32 off) and fp32 output for both squares.
    vendor = {}
    if not args.no_vendor:
        tf32 = torch.backends.cuda.matmul.allow_tf32
        torch.backends.cuda.matmul.allow_tf32 = False
        vf = lambda i: torch.mm(A, B, out=C)
        ramp(vf, stream, args.ramp_ms)
        vendor["square_4096_f32"] = vendor_entry("torch.mm(A, B, out=C), fp32, TF32 off",
                                                 time_launches(vf, args.steps, stream), ms)
        try:
            vb = lambda i: torch.mm(Ab, Bb, out_dtype=torch.float32)
            ramp(vb, stream, args.ramp_ms)
            vendor["square_4096_bf16"] = vendor_entry("torch.mm(A, B, out_dtype=torch.float32), bf16 in",
                                                      time_launches(vb, args.steps, stream), msb)
        except (TypeError, RuntimeError) as e:  # out_dtype is not in every torch build
            vendor["square_4096_bf16"] = {"error": str(e)[:160]}
        vbb = lambda i: torch.mm(Ab, Bb, out=Cb)
        ramp(vbb, stream, args.ramp_ms)
        vendor["square_4096_bf16_out_bf16"] = vendor_entry("torch.mm(A, B, out=C), bf16 in and out",
                                                           time_launches(vbb, args.steps, stream), msbb)
        torch.backends.cuda.matmul.allow_tf32 = tf32
        log(f"vendor squares: {vendor}")
    del Ab, Bb, Cb

    # ---- narrow fp16 linear 16×4096×4096, cold weights -----------------------------------
    log("narrow fp16 16x4096x4096: generating inputs")
    nc = inputs.workload_fp16_narrow()
    X = to_dev(nc.X, "f16")
    W0 = to_dev(nc.W, "f16")
    Ws = [W0] + [W0.clone() for _ in range(COLD_COPIES - 1)]
    Y = torch.empty((nc.M, nc.N), dtype=torch.float16, device=dev)
    nplan = tlgemm.Plan.create(nc.M, nc.N, nc.K, "f16", "f16", "NK")
    nws_bytes = nplan.workspace_size
    nws = torch.zeros(max(nws_bytes, 1), dtype=torch.uint8, device=dev)  # zero before first use
    run_n = lambda i: nplan.run_ptrs(X.data_ptr(), Ws[i % COLD_COPIES].data_ptr(), 0, Y.data_ptr(),
                                     nws.data_ptr() if nws_bytes else 0, nws_bytes, stream.cuda_stream)
    run_n(0)
    torch.cuda.synchronize()
    n_err = None if args.no_parity else sampled_parity(nc, to_f64(Y))
    ramp(run_n, stream, args.ramp_ms)
    n_ms = time_launches(run_n, args.narrow_launches, stream)
    warm_ms = time_launches(lambda i: run_n(0), args.narrow_launches, stream)
    n_bytes = nc.M * nc.K * 2 + nc.N * nc.K * 2 + nc.M * nc.N * 2
    n_gbs = n_bytes / (n_ms * 1e-3) / 1e9
    log(f"narrow fp16: {nplan.describe()} cold {n_ms * 1e3:.2f} us ({n_gbs:.0f} GB/s), warm {warm_ms * 1e3:.2f} us, "
        f"parity {n_err}")
    if not args.no_vendor:
        vn = lambda i: torch.nn.functional.linear(X, Ws[i % COLD_COPIES])
        ramp(vn, stream, args.ramp_ms)
        vendor["narrow_16x4096x4096_f16"] = vendor_entry(
            f"F.linear(X, W) over the same {COLD_COPIES} rotated weight copies",
            time_launches(vn, args.narrow_launches, stream), n_ms)

    extra = {}
    if not args.no_extra:
        log("ceilings: launch floor, plain 32 MiB read, MFMA issue rate")
        extra["ceilings"] = bench_ceilings(torch, dev, stream, Ws)
        del Ws, W0
        log("fp32 linear 128x768x768 + bias")
        extra["linear_128x768x768_f32"] = bench_c1(torch, dev, stream, args.no_parity)
        log("GPT-2 layer at M=128, fp32")
        extra["gpt2_layer_m128_f32"] = bench_c3(torch, dev, stream, args.no_parity)
        for dt in ("f32", "bf16"):
            log(f"GPT-2 stack at M=8192, {dt}")
            extra[f"gpt2_stack_m8192_{dt}"] = bench_c5(torch, dev, stream, dt, args.no_parity,
                                                       vendor=not args.no_vendor)
            if not args.no_vendor:
                vendor[f"gpt2_stack_m8192_{dt}"] = extra[f"gpt2_stack_m8192_{dt}"]["vendor_library"]
            torch.cuda.empty_cache()
        for dt in ("f32", "bf16"):
            log(f"GPT-2-small forward, 12 blocks, {dt}")
            extra[f"gpt2_forward_12x_b64_t128_{dt}"] = bench_gpt2_forward(torch, dev, stream, dt, args.no_parity)
            torch.cuda.empty_cache()
        for dt in ("f32", "bf16"):
            log(f"GPT-2 layer ops (LayerNorm, attention), {dt}")
            extra[f"gpt2_layer_ops_{dt}"] = bench_layer_ops(torch, dev, stream, dt, args.no_parity)
        for dt in ("f32", "bf16"):
            log(f"GPT-2 backward GEMMs at 8192 tokens, {dt}")
            extra[f"gpt2_backward_t8192_{dt}"] = bench_backward(torch, dev, stream, dt, args.no_parity)
            torch.cuda.empty_cache()
    clocks_after = read_clocks(torch)

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline: timing the oracle on every workload (whole outputs or row samples)")
        cpu = cpu_baseline()
        gpu_s = {"square_4096_f32": ms * 1e-3, "square_4096_bf16": msb * 1e-3,
                 "narrow_16x4096x4096_f16": n_ms * 1e-3}
        if "linear_128x768x768_f32" in extra:
            gpu_s["linear_128x768x768_f32"] = extra["linear_128x768x768_f32"]["warm_us"] * 1e-6
            gpu_s["gpt2_layer_m128_f32"] = extra["gpt2_layer_m128_f32"]["layer_warm_us"] * 1e-6
            for dt in ("f32", "bf16"):
                gpu_s[f"gpt2_stack_m8192_{dt}"] = extra[f"gpt2_stack_m8192_{dt}"]["pass_ms"] * 1e-3
        for k, v in cpu["per_workload"].items():
            if k in gpu_s:
                v["gpu_s"] = gpu_s[k]
                v["gpu_over_oracle_all_cores"] = round(v["all_cores_s"] / gpu_s[k], 1)

    tol32, tol16 = 1e-5, 1e-2
    out = {
        "metric": METRIC,
        "value": round(sq_tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_ramp_ms": args.ramp_ms,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "fp32 GEMM C=A.B, M=N=K=4096, row-major A[M][K] and B[K][N], U(-1,1), warm",
                   "M": sq.M, "N": sq.N, "K": sq.K, "layout": "KN", "plan": plan.describe()},
        "roofline": {"bound": "mfma", "achieved": round(sq_tflops, 3), "peak": PEAK_F32_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(sq_tflops / PEAK_F32_TFLOPS, 4),
                     "traffic": measured_traffic("tiled_f32", tile_str(plan)),
                     "traffic_unit": "bytes per launch (L2<->memory, rocprofv3 FETCH_SIZE+WRITE_SIZE)",
                     "algorithmic_bytes_per_launch": 3 * sq.M * sq.N * 4,
                     "kernel": f"tiled_kernel fp32 {plan.info.tile_m}x{plan.info.tile_n}x{plan.info.tile_k}",
                     "algorithmic_flops_per_launch": sq.flops,
                     **clock_adjusted(extra.get("ceilings"), sq_tflops, PEAK_F32_TFLOPS, "f32")},
        "cpu_baseline": cpu,
        "parity": {"square_f32_err": sq_err, "square_f32_pass": None if sq_err is None else sq_err <= tol32,
                   "square_bf16_err": sqb_err, "narrow_f16_err": n_err,
                   "narrow_f16_pass": None if n_err is None else n_err <= tol16,
                   "measure": "max|err|/max|ref| on sampled outputs vs the CPU oracle"},
        "square_bf16": {"us": round(msb * 1e3, 2), "TFLOP/s": round(sqb.flops / (msb * 1e-3) / 1e12, 2),
                        "frac_mfma_peak": round(sqb.flops / (msb * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                        **clock_adjusted(extra.get("ceilings"), sqb.flops / (msb * 1e-3) / 1e12, PEAK_BF16_TFLOPS,
                                         "bf16"),
                        **l2_roofline(extra.get("ceilings"), planb, sqb, msb),
                        "plan": planb.describe(),
                        "bf16_out": {"us": round(msbb * 1e3, 2),
                                     "TFLOP/s": round(sqb.flops / (msbb * 1e-3) / 1e12, 2),
                                     "frac_mfma_peak": round(sqb.flops / (msbb * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                                     "parity_err": sqbb_err, "plan": planbb.describe()}},
        "narrow_fp16": {"workload": "fp16 linear Y=X.W^T, M=16, K=4096, N=4096, W out x in, fp16 out, cold W "
                                    f"({COLD_COPIES} rotated copies)",
                        "us": round(n_ms * 1e3, 3), "warm_us": round(warm_ms * 1e3, 3),
                        "GB/s": round(n_gbs, 1),
                        **({"frac_of_measured_cold_read": round(n_gbs / extra["ceilings"]["read_cold_GB/s"], 4),
                            "measured_cold_read_GB/s": extra["ceilings"]["read_cold_GB/s"]}
                           if (extra.get("ceilings") or {}).get("read_cold_GB/s") else {}),
                        "roofline": {"bound": "hbm", "achieved": round(n_gbs, 1), "peak": PEAK_HBM_GBS,
                                     "unit": "GB/s", "frac": round(n_gbs / PEAK_HBM_GBS, 4),
                                     "traffic": measured_traffic("stream_f16", tile_str(nplan)),
                                     "kernel": f"stream kernel fp16 {nplan.info.tile_m}x{nplan.info.tile_n}, "
                                               f"{nplan.info.threads // 64} waves over K"
                                               + (", each wave's K range of the weight rows in LDS" if "load=direct" in nplan.describe() else ""),
                                     "algorithmic_bytes_per_launch": n_bytes},
                        "timing": "HIP events over back-to-back launches (includes launch gaps)",
                        "plan": nplan.describe()},
        "vendor_library": {"note": "context, not a baseline: the same workloads through torch (hipBLASLt or "
                                   "rocBLAS) on this GPU, timed like this library's; ours_speedup = vendor time / "
                                   "ours", **vendor} if vendor else None,
        "clocks": {"before": clocks_before, "after": clocks_after,
                   "state": "UNPINNED" + (" (changed during the run)" if clocks_before != clocks_after else "")},
    }
    out.update(extra)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
