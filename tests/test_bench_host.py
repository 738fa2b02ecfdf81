"""Host logic of bench.py (CPU): the code hash that keys the counter-derived traffic, and the
reduction of rocprofv3 counter and kernel-statistics files into the committed summaries."""
import csv
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_code_text_ignores_comments_and_layout():
    a = "int f(int x) {  // doubles x\n  /* a\n block */ return 2 * x;\n}\n"
    b = "int f(int x) { return 2 * x; }"
    assert bench.code_text(a) == bench.code_text(b)
    assert bench.code_text(a) != bench.code_text(b.replace("2 *", "3 *"))
    assert "doubles" not in bench.code_text(a) and "block" not in bench.code_text(a)


def test_source_hash_tracks_the_kernel_sources(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("__global__ void k() { /* v1 */ }\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h1 = bench.source_hash(["k.hip"])
    src.write_text("__global__ void k() {   // v2, reworded\n}\n")
    assert bench.source_hash(["k.hip"]) == h1          # comment and layout edits
    src.write_text("__global__ void k() { int a; }\n")
    assert bench.source_hash(["k.hip"]) != h1          # a code edit


def test_every_kernel_source_exists():
    for p in bench.KERNEL_SOURCES:
        assert os.path.exists(os.path.join(ROOT, p)), p


def _counter_csv(d, counter, values):
    """A counter_collection.csv with one row per (kernel name, value)."""
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "p_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, v in values:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": v})


def test_summarize_pmc_calibrates_and_sums_each_pass(tmp_path):
    # the calibration copy reads FETCH 32768 KiB (scale 2) and writes WRITE 65536 KiB
    # (scale 1); the GEMM pass has two dispatches per call averaged; the columns pass is its
    # one kernel, not the scratch fill (cols[0]) that longer column passes launch
    gemm = "void halo::gemm_kernel<0, 0, 0, 2, false, 128, 4>(halo::GemmPair)"
    # (the fp32-input instantiation of the same kernel is its own pass)
    cols = ["void halo::fill_zero_kernel(float*, long)",
            "void halo::fq_cols2_kernel<256, 0, false, false, false>(halo::ColsProb, halo::ColsProb, long, long)",
            "void halo::fq_cols2_kernel<256, 0, false, false, true>(halo::ColsProb, halo::ColsProb, long, long)"]
    neg = "void at::native::neg_kernel_impl"
    _counter_csv(tmp_path / "f", "FETCH_SIZE",
                 [(gemm, 1000.0), (gemm, 3000.0), (cols[0], 1.0), (cols[1], 99.0),
                  (cols[2], 7.0), (neg, 32768.0)])
    _counter_csv(tmp_path / "w", "WRITE_SIZE",
                 [(gemm, 500.0), (gemm, 500.0), (cols[0], 2.0), (cols[1], 48.0),
                  (cols[2], 5.0), (neg, 65536.0)])
    res, text = bench.summarize_pmc(str(tmp_path / "f"), str(tmp_path / "w"), "cmd")
    assert res["fetch_scale"] == pytest.approx(2.0) and res["write_scale"] == pytest.approx(1.0)
    b = res["bytes_per_launch"]
    assert b["gemm_i8_4096"] == int(round(2000.0 * 1024 * 2 + 500.0 * 1024))
    assert b["fq_cols_4096"] == int(round(99.0 * 1024 * 2 + 48.0 * 1024))
    assert b["fq_cols_f32_4096"] == int(round(7.0 * 1024 * 2 + 5.0 * 1024))
    assert "fq_rows_4096" not in b  # no counters for it: left out, never zero
    assert res["kernel_source_hash"] == bench.source_hash(bench.KERNEL_SOURCES)
    assert text.startswith("command: cmd")


def test_summarize_stats_orders_by_total_time(tmp_path):
    p = tmp_path / "kt_kernel_stats.csv"
    with open(p, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "TotalDurationNs", "AverageNs",
                                          "Percentage", "MinNs", "MaxNs"])
        w.writeheader()
        w.writerow(dict(Name="small", Calls=2, TotalDurationNs=2000, AverageNs=1000,
                        Percentage=10.0, MinNs=900, MaxNs=1100))
        w.writerow(dict(Name="big", Calls=1, TotalDurationNs=18000, AverageNs=18000,
                        Percentage=90.0, MinNs=18000, MaxNs=18000))
    text = bench.summarize_stats(str(p), "cmd")
    lines = text.splitlines()
    assert lines[0] == "command: cmd"
    body = [l for l in lines if l.endswith("big") or l.endswith("small")]
    assert body[0].endswith("big") and "18.00" in body[0]
    assert body[1].endswith("small") and "1.00" in body[1]


def test_algorithmic_bytes():
    # 3 B per element (bf16 read, one code byte written) plus one fp32 scale per vector
    assert bench.FQ_BYTES == 4096 * 4096 * 3 + 4 * 4096
    assert bench.LARGE_BYTES == 16384 * 14336 * 3 + 4 * 16384
    assert bench.GEMM_BYTES == 2 * 4096 * 4096 + 2 * 4096 * 4096 + 4 * 8192
    assert np.isclose(bench.STEP_GOP, 3 * 2 * 4096 ** 3 / 1e9)


def test_summarize_counters_means_and_derived(tmp_path):
    gemm = "void halo::gemm_kernel<0, 0, 0, 2, false, 128, 4>(halo::GemmPair)"
    d = tmp_path / "a"
    os.makedirs(d)
    with open(d / "p_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Grid_Size", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for v in (100.0, 300.0):  # two calls of the single product
            w.writerow(dict(Kernel_Name=gemm, Grid_Size=bench.GEMM_GRID,
                            Counter_Name="SQ_VALU_MFMA_BUSY_CYCLES", Counter_Value=v * 1024))
            w.writerow(dict(Kernel_Name=gemm, Grid_Size=bench.GEMM_GRID,
                            Counter_Name="GRBM_GUI_ACTIVE", Counter_Value=8 * 400.0))
        # the paired products (twice the grid) must not mix in
        w.writerow(dict(Kernel_Name=gemm, Grid_Size=2 * bench.GEMM_GRID,
                        Counter_Name="SQ_VALU_MFMA_BUSY_CYCLES", Counter_Value=9e9))
    text = bench.summarize_counters([str(d)], ["cmd a"])
    assert text.startswith("command (pass 1): cmd a")
    assert "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x that) = 50.0 %" in text
    means = bench._counter_means(str(d))
    assert means["gemm_i8_4096"]["SQ_VALU_MFMA_BUSY_CYCLES"] == pytest.approx(200.0 * 1024)
    assert means["gemm_i8_pair_4096"]["SQ_VALU_MFMA_BUSY_CYCLES"] == pytest.approx(9e9)


def test_workload_passes_follow_the_configuration():
    import synth
    fq, prods = bench.workload_passes(synth.WORKLOADS["c4_fwdbwd_8192x4096x11008_bf16_b128_i8"])
    assert [p[0] for p in fq] == ["x_rows", "w_rows", "dy_rows", "w_cols", "dy_cols", "x_cols"]
    assert prods == [("y", "x_rows", "w_rows"), ("dx", "dy_rows", "w_cols"),
                     ("dw", "dy_cols", "x_cols")]
    # every product's operands come from passes along the same contraction dimension
    axis_src = {p[0]: (p[1], p[2]) for p in fq}
    assert axis_src["dy_cols"] == ("dy", 1) and axis_src["x_cols"] == ("x", 1)
    fq, prods = bench.workload_passes(synth.WORKLOADS["c1_fwd_256x1024x1024_f32_b1024_i8"])
    assert len(fq) == 2 and prods == [("y", "x_rows", "w_rows")]
