"""Host logic of bench.py, on the CPU: the kernel names and lane-op model it reports,
the summaries it makes of rocprofv3 output, the stored traffic files' source gating
and the one-GPU rule.  No GPU and no library call."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_head_kernel_names_follow_the_library_choice():
    # the 243M-shape bf16 line takes the persistent form; fp32 rows and small products
    # take one workgroup per token
    assert bench.head_kernel_name(8192, 50304, 1024, True) == "head_stream_kernel"
    assert bench.head_kernel_name(8192, 50304, 1024, False) == "head_estimate_kernel"
    assert bench.head_kernel_name(4096, 8192, 512, False) == "head_estimate_kernel"
    assert bench.head_kernel_name(4096, 8192, 512, True) == "head_estimate_kernel"   # V <= 8192
    assert bench.head_kernel_name(16, 50304, 64, True) == "head_estimate_kernel"     # small product
    assert bench.head_kernel_name(8192, 50301, 1024, True) == "head_estimate_kernel"  # V not a multiple of 8
    assert bench.subset_kernel_name(8192) == "head_subset_kernel"
    assert bench.subset_kernel_name(16384) == "head_subset_kernel"
    assert "+" in bench.subset_kernel_name(16385)


def test_taylor_degree_and_lane_op_model():
    # the degrees the workloads run at (sigma 5e-3: 3, 1e-2: 4) and the model's count
    assert bench.head_taylor_degree(5e-3) == 3
    assert bench.head_taylor_degree(1e-2) == 4
    assert bench.head_taylor_degree(0.5) == 6
    assert bench.head_lane_ops_per_channel_draw(3) == pytest.approx(19.5)
    assert bench.head_lane_ops_per_channel_draw(4) == pytest.approx(20.5)


def _write_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def test_trace_summary_reads_stats_and_launch_shapes(tmp_path, capsys):
    _write_csv(tmp_path / "x_kernel_stats.csv", [
        {"Name": "dust::k1(int)", "Calls": "2", "TotalDurationNs": "3000", "AverageNs": "1500", "MinNs": "1000",
         "MaxNs": "2000", "Percentage": "75.0"},
        {"Name": "other(int)", "Calls": "1", "TotalDurationNs": "1000", "AverageNs": "1000", "MinNs": "1000",
         "MaxNs": "1000", "Percentage": "25.0"}])
    _write_csv(tmp_path / "x_kernel_trace.csv", [
        {"Kernel_Name": "dust::k1(int)", "Grid_Size_X": "1024", "Grid_Size_Y": "1", "Grid_Size_Z": "2",
         "Workgroup_Size_X": "256", "Workgroup_Size_Y": "1", "Workgroup_Size_Z": "1", "VGPR_Count": "64",
         "Accum_VGPR_Count": "0", "LDS_Block_Size": "4096", "Scratch_Size": "0"}])
    bench.trace_summary(type("A", (), {"trace_summary": str(tmp_path)})())
    out = capsys.readouterr().out
    assert "| `dust::k1(int)` | 2 | 3.0 | 1.5 | 1.0 | 2.0 | 75.0 |" in out
    assert "grid 1024x1x2, workgroup 256x1x1, VGPR 64, AGPR 0, LDS 4096 B, scratch 0 B" in out
    assert "other(int)`:" not in out   # launch shapes of library kernels only


def test_counter_summary_sums_a_dispatch_and_averages_dispatches(tmp_path, capsys):
    rows = []
    for disp, parts in ((1, (10.0, 20.0)), (2, (30.0, 40.0))):   # two instances per dispatch
        for v in parts:
            rows.append({"Dispatch_Id": str(disp), "Kernel_Name": "dust::k(int)", "Counter_Name": "SQ_WAVES",
                         "Counter_Value": str(v)})
    rows.append({"Dispatch_Id": "3", "Kernel_Name": "copy(int)", "Counter_Name": "SQ_WAVES", "Counter_Value": "5"})
    d = tmp_path / "run"
    d.mkdir()
    _write_csv(d / "p_counter_collection.csv", rows)
    bench.counter_summary([str(d)])
    out = capsys.readouterr().out
    assert "### `dust::k`" in out
    assert "| SQ_WAVES | 50 | 2 |" in out   # (10 + 20 + 30 + 40) / 2 dispatches
    assert "copy" not in out


def test_traffic_files_are_gated_by_their_sources():
    for name in os.listdir(os.path.join(ROOT, "profiles")):
        if not name.startswith("traffic_"):
            continue
        t = json.load(open(os.path.join(ROOT, "profiles", name)))
        assert t["kernel"] in bench.KERNEL_SOURCES
        assert t["bytes_per_launch"] == pytest.approx(t["fetch"]["bytes"] + t["write"]["bytes"])
        assert len(t["commands"]) == 5 and all("rocprofv3 --pmc" in c for c in t["commands"][:4])
        # a file taken on other sources reports no traffic
        assert (bench.load_traffic(t["kernel"], t["workload"], t["subset_m"]) is None) == \
            (t["sources_sha256"] != bench.sources_digest(t["kernel"]))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
