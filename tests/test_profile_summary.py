"""The rocprofv3 summariser on small synthetic CSVs (CPU only): the dispatch
labels, the copy-probe calibration of FETCH_SIZE / WRITE_SIZE, the derived
MFMA-busy and LDS-conflict columns, and the kernel-trace table."""

import csv
import json

import pytest

from sparse_attention_context_amd import profile_summary as ps

KERNELS = ["void at::native::elementwise_kernel<cast>(int)",
           "void isa::isa_pool_kernel<unsigned short, 128>(isa::PoolArgs)",
           "isa::isa_flash_pps_kernel(isa::FlashArgs)",
           "void isa::isa_flash_pp_kernel<0, 0, 128>(isa::FlashArgs)",
           "void at::native::vectorized_elementwise_kernel<4, FillFunctor>(int)",
           "void at::native::vectorized_elementwise_kernel<4, MulFunctor>(int)"]


def _write_run(d, counters):
    d.mkdir(parents=True)
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, name in enumerate(KERNELS):
            for cname, vals in counters.items():
                w.writerow([i + 1, name, cname, vals[i]])


def test_counter_summary_labels_and_calibration(tmp_path):
    gib_kib = (1 << 30) / 1024
    # the copy probe (last) reads 1 GiB but FETCH_SIZE reports half of it
    _write_run(tmp_path / "p1", {"FETCH_SIZE": [100, 1000, 2000, 3000, 10, gib_kib / 2]})
    _write_run(tmp_path / "p2", {"WRITE_SIZE": [100, 50, 60, 70, gib_kib, gib_kib]})
    _write_run(tmp_path / "p3", {"SQ_VALU_MFMA_BUSY_CYCLES": [0, 0, 512, 0, 0, 0],
                                 "GRBM_GUI_ACTIVE": [8, 8, 8, 8, 8, 8]})
    text = ps.counters(str(tmp_path))
    assert "fetch_scale 2.0000" in text and "write_scale 1.0000" in text
    assert ps.sources_digest() in text
    rows = {ln[:48].strip(): ln[48:].split() for ln in text.splitlines() if ln and not ln.startswith("#")}
    assert "torch input cast (outside the layer) #1" in rows
    assert "copy probe: torch.mul(src, 1.0, out=dst), 1 GiB" in rows
    assert "torch.ones fill, 1 GiB out #1" in rows
    pps = rows["isa_flash_pps_kernel full route"]
    # HBM_MB = (2000 KiB * 2 + 60 KiB) * 1024 / 1e6; MFMA busy = 512 / (8 / 8 * 1024) = 50 %
    assert float(pps[2]) == pytest.approx((2000 * 2 + 60) * 1024 / 1e6, abs=0.05)
    assert float(pps[3]) == pytest.approx(50.0)
    assert "isa_pool_kernel<bf16,128>" in rows and "isa_flash_pp_kernel<0,0,128> dense" in rows


def test_counter_runs_must_dispatch_the_same_kernels(tmp_path):
    _write_run(tmp_path / "p1", {"FETCH_SIZE": [1, 1, 1, 1, 1, 1]})
    (tmp_path / "p2").mkdir()
    with open(tmp_path / "p2" / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, name in enumerate(reversed(KERNELS)):
            w.writerow([i + 1, name, "WRITE_SIZE", 1])
    with pytest.raises(SystemExit):
        ps.counters(str(tmp_path))


def test_trace_table_and_bench_figures(tmp_path):
    stats = tmp_path / "run_kernel_stats.csv"
    with open(stats, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage"])
        w.writerow(["isa::isa_flash_pps_kernel(isa::FlashArgs)", 10, 9_000_000, 900_000, 90])
        w.writerow(["void isa::isa_pool_kernel<unsigned short, 128>(isa::PoolArgs)", 10, 1_000_000, 100_000, 10])
    bench = tmp_path / "bench.json"
    bench.write_text("log line\n" + json.dumps({
        "ms_per_step": 1.2, "timing": {"n": 20, "warm_median_ms": 1.1},
        "roofline": {"avg_launch_ms": 0.9, "achieved": 1050.0, "unit": "TFLOP/s", "frac": 0.42, "peak": 2500.0},
        "other_rooflines": [], "stage_ms": {"full": 0.9}}) + "\n")
    text = ps.trace(str(stats), str(bench))
    lines = text.splitlines()
    assert lines[1].startswith("isa::isa_flash_pps_kernel") and "900.00" in lines[1] and "90.00" in lines[1]
    assert "ms_per_step 1.2" in text and "frac 0.42" in text
