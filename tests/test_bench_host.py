"""Host logic of bench.py on the CPU: the rocprofv3 summarisers that write the committed
profiles, the derived roofline figures, and the one-GPU guard.  No GPU and no torch GPU calls."""
import csv
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402

TRACE_COLS = ["Kernel_Name", "Dispatch_Id", "Workgroup_Size_X", "Workgroup_Size_Y", "Workgroup_Size_Z",
              "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z", "Start_Timestamp", "End_Timestamp"]
SQUARE = "void tlg::tiled_kernel<0, 0, 1, 0u, 256, 256, 16, 2, 4, true, false, 0, false>(void const*)"
BWD = "void tlg::tiled_kernel<0, 0, 1, 0u, 256, 256, 16, 2, 4, true, false, 0, false>(void const*)"


def write_csv(path, cols, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(cols)
        w.writerows(rows)


def trace_row(name, disp, threads, grid_wg, dur_ns, t0=0):
    return [name, disp, threads, 1, 1, grid_wg * threads, 1, 1, t0, t0 + dur_ns]


def test_rocprof_summary_keeps_grids_apart_and_drops_runtime_kernels(tmp_path):
    # one template at two grids (the square and a backward product share a name) must not pool
    rows = [trace_row(SQUARE, i, 512, 256, 900_000 + 1000 * i) for i in range(5)]
    rows += [trace_row(BWD, 10 + i, 512, 96, 200_000) for i in range(3)]
    rows += [trace_row("void at::native::vectorized_elementwise_kernel<4>(int)", 20, 256, 64, 5_000)]
    rows += [trace_row("__amd_rocclr_copyBuffer", 21, 256, 256, 7_000)]
    rows += [trace_row("Cijk_Ailk_Bljk_BBS_BH_MT256x256x64_MI16x16x1", 22, 256, 256, 100_000)]  # vendor GEMM
    write_csv(str(tmp_path / "run" / "x_kernel_trace.csv"), TRACE_COLS, rows)
    md = bench.rocprof_summary(str(tmp_path), [])
    table = [l for l in md.splitlines() if l.startswith("| `")]
    assert len(table) == 2  # runtime, torch and vendor BLAS kernels left out
    sq = [l for l in table if "| 256x1x1 |" in l]
    bw = [l for l in table if "| 96x1x1 |" in l]
    assert len(sq) == 1 and len(bw) == 1
    cells = [c.strip() for c in sq[0].split("|")]
    assert cells[3] == "5" and float(cells[4]) == pytest.approx(902.0)  # launches, median µs
    assert float(cells[7]) == pytest.approx(900.0)  # min µs
    assert [c.strip() for c in bw[0].split("|")][3] == "3"
    assert "(void const*)" not in md  # parameter list dropped, template arguments kept


def test_rocprof_summary_segments_split_in_dispatch_order(tmp_path):
    # 2 parity launches, a ramp of unknown length ('*'), then 4 timed launches
    durs = [50_000, 50_000] + [20_000] * 7 + [10_000] * 4
    rows = [trace_row(SQUARE, i, 512, 256, d, t0=1000 * i) for i, d in enumerate(durs)]
    rows.reverse()  # file order is not dispatch order
    write_csv(str(tmp_path / "x_kernel_trace.csv"), TRACE_COLS, rows)
    name = SQUARE[:SQUARE.rindex("(")]
    md = bench.rocprof_summary(str(tmp_path), [SQUARE + "@256x1x1=2,*,4"])
    runs = [l for l in md.splitlines() if l.startswith("| 0 |") or l.startswith("| 1 |") or l.startswith("| 2 |")]
    assert [r.split("|")[2].strip() for r in runs] == ["2", "7", "4"]
    assert [float(r.split("|")[3]) for r in runs] == [50.0, 20.0, 10.0]
    assert name in md
    with pytest.raises(SystemExit):  # counts that do not add up are refused
        bench.rocprof_summary(str(tmp_path), [SQUARE + "@256x1x1=2,3"])
    with pytest.raises(SystemExit):
        bench.rocprof_summary(str(tmp_path), [SQUARE + "@256x1x1=*,*"])


PMC_COLS = ["Kernel_Name", "Workgroup_Size", "Grid_Size", "Counter_Name", "Counter_Value"]


def test_pmc_summary_calibrates_on_the_32mib_copy(tmp_path):
    copy = "__amd_rocclr_copyBuffer"
    k = "void tlg::stream_dl_kernel<1, 1, 0u, 8>(void const*)"
    # the counters read half the true bytes for the copy: every figure is scaled by 2
    write_csv(str(tmp_path / "f" / "a_counter_collection.csv"), PMC_COLS,
              [[copy, 256, 256 * 256, "FETCH_SIZE", 16384.0]] * 3 + [[k, 512, 256 * 512, "FETCH_SIZE", 16500.0]] * 5)
    write_csv(str(tmp_path / "w" / "a_counter_collection.csv"), PMC_COLS,
              [[copy, 256, 256 * 256, "WRITE_SIZE", 16384.0]] * 3 + [[k, 512, 256 * 512, "WRITE_SIZE", 32.0]] * 5)
    alg = 33_816_576
    md = bench.pmc_summary(str(tmp_path / "f"), str(tmp_path / "w"), [k[:k.rindex("(")] + f"@256x1x1={alg}"])
    assert "scaled by 2.000" in md
    row = [l for l in md.splitlines() if l.startswith("| `")][0].split("|")
    scaled = float(row[6])
    assert scaled == pytest.approx((16500.0 + 32.0) * 1024 * 2, rel=1e-6)
    assert float(row[8]) == pytest.approx(scaled / alg, abs=0.01)
    with pytest.raises(SystemExit):  # a row that names no kernel of the run
        bench.pmc_summary(str(tmp_path / "f"), str(tmp_path / "w"), ["void tlg::nothing@1x1x1=1"])


def test_counter_summary_derives_clock_and_mfma_busy(tmp_path):
    k = SQUARE
    cyc = 2.2e6  # core cycles of one dispatch; the counter sums 8 XCDs
    rows = [[k, 512, 256 * 512, "GRBM_GUI_ACTIVE", 8 * cyc]] * 3
    rows += [[k, 512, 256 * 512, "SQ_VALU_MFMA_BUSY_CYCLES", 0.95 * cyc * 1024]] * 3
    rows += [[k, 512, 256 * 512, "SQ_LDS_BANK_CONFLICT", 10.0], [k, 512, 256 * 512, "SQ_LDS_IDX_ACTIVE", 100.0]]
    write_csv(str(tmp_path / "a_counter_collection.csv"), PMC_COLS, rows)
    dur_ns = 1_000_000  # 1 ms -> 2200 MHz
    write_csv(str(tmp_path / "a_kernel_trace.csv"), TRACE_COLS, [trace_row(k, i, 512, 256, dur_ns) for i in range(3)])
    md = bench.counter_summary([str(tmp_path)], [k[:k.rindex("(")] + "@256x1x1"])
    head = [c.strip() for c in md.splitlines()[0].split("|")]
    row = [c.strip() for c in md.splitlines()[2].split("|")]
    got = dict(zip(head, row))
    assert float(got["median µs"]) == pytest.approx(1000.0)
    assert float(got["core MHz"]) == pytest.approx(2200.0, rel=1e-3)
    assert float(got["MFMA busy"]) == pytest.approx(0.95, abs=1e-3)
    assert float(got["LDS conflict share"]) == pytest.approx(0.1, abs=1e-3)


def test_clock_adjusted_and_vendor_entry():
    ceil = {"sclk_MHz_under_mfma_f32": 2100.0}
    r = bench.clock_adjusted(ceil, 150.0, bench.PEAK_F32_TFLOPS, "f32")
    assert r["peak_clock_adjusted"] == pytest.approx(bench.PEAK_F32_TFLOPS * 2100 / bench.PEAK_SCLK_MHZ, abs=0.01)
    assert r["frac_clock_adjusted"] == pytest.approx(150.0 / r["peak_clock_adjusted"], abs=1e-4)
    assert bench.clock_adjusted(None, 1.0, 1.0, "f32") == {}
    assert bench.clock_adjusted({}, 1.0, 1.0, "bf16") == {}
    v = bench.vendor_entry("x", 0.019, 0.008)
    assert v["us"] == 19.0 and v["ours_us"] == 8.0 and v["ours_speedup"] == pytest.approx(19 / 8, abs=1e-3)


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_peaks_are_the_datasheet_figures():
    assert bench.PEAK_F32_TFLOPS == pytest.approx(157.3, abs=0.1)
    assert bench.PEAK_HBM_GBS == pytest.approx(8000.0)
    assert 2400 <= bench.PEAK_BF16_TFLOPS <= 2600
    assert np.isfinite(bench.PEAK_SCLK_MHZ) and bench.PEAK_SCLK_MHZ == 2400


def test_linear_floor_takes_the_larger_of_the_two_bounds():
    """128×768×768 fp32 is MFMA-bound (2·128·768² flops at 157.3 TF/s = 0.960 µs against 3.15 MB at 8 TB/s);
    one row against a 4096² weight is HBM-bound (67.1 MB at 8 TB/s = 8.39 µs against 0.21 µs of MFMA work)."""
    from types import SimpleNamespace as NS
    c1 = NS(M=128, N=768, K=768, flops=2 * 128 * 768 * 768)
    assert bench.linear_floor_us(c1) == pytest.approx(2 * 128 * 768 * 768 / 157.3e12 * 1e6)
    row = NS(M=1, N=4096, K=4096, flops=2 * 4096 * 4096)
    assert bench.linear_floor_us(row) == pytest.approx(4 * (4096 + 4096 * 4096 + 4096 + 4096) / 8000e9 * 1e6)
