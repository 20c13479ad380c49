"""Host-side logic of bench.py, on the CPU: the one-GPU guard, the
rocprofv3 summarizers that turn kernel traces, marker traces and counter
collections into the tables under profiles/, the HBM-traffic calibration
against a device copy, and the source-hash gate on committed counters.

The CSV inputs are small synthetic files with rocprofv3's column names;
every expected figure below is worked out by hand from them."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def table_rows(text):
    """Data rows of every markdown table in text, as lists of cells."""
    out = []
    for line in text.splitlines():
        if line.startswith("|") and not set(line.replace("|", "").strip()) <= set("-: "):
            out.append([c.strip() for c in line.strip("|").split("|")])
    return out


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_summarize_profile_kernel_trace(tmp_path, capsys):
    """Durations are End - Start in ns, reported in us per (kernel, grid);
    the dispatch range a:b averages launches a..b-1 in start order."""
    name = "void detred::lds::wide_gemm_kernel<LdsTile<192, 128, 2, 4>, 4, false>(detred::GemmArgs)"
    rows = []
    # five launches of 10, 20, 30, 40, 50 us, listed out of start order
    for i, us in [(3, 40), (0, 10), (4, 50), (1, 20), (2, 30)]:
        start = 1_000_000 * i
        rows.append([name, 1261568, start, start + us * 1000])
    rows.append(["void detred::rmsnorm_kernel<float>(float*)", 65536, 9_000_000, 9_006_000])
    write_csv(str(tmp_path / "run" / "run_kernel_trace.csv"),
              ["Kernel_Name", "Grid_Size", "Start_Timestamp", "End_Timestamp"], rows)
    bench.summarize_profile(str(tmp_path), "1:3")
    got = {r[0]: r for r in table_rows(capsys.readouterr().out) if r[0].startswith("`")}
    wide = got["`wide_gemm_kernel<LdsTile<192, 128, 2, 4>, 4, false>`"]
    assert wide[1:] == ["1261568", "5", "30.00", "10.00", "50.00", "25.00"]
    norm = got["`rmsnorm_kernel<float>`"]
    assert norm[1:] == ["65536", "1", "6.00", "6.00", "6.00", "-"]


def test_summarize_profile_counters(tmp_path, capsys):
    """A counter's rows of one dispatch (one per XCD or instance) are added,
    then the per-dispatch sums are averaged over dispatches."""
    k = "void detred::tree_combine_kernel<8>(float const*)"
    rows = [[k, 1048576, "GRBM_GUI_ACTIVE", 100, 1], [k, 1048576, "GRBM_GUI_ACTIVE", 300, 1],
            [k, 1048576, "GRBM_GUI_ACTIVE", 200, 2], [k, 1048576, "GRBM_GUI_ACTIVE", 400, 2],
            [k, 1048576, "SQ_WAVES", 7, 1], [k, 1048576, "SQ_WAVES", 9, 2]]
    write_csv(str(tmp_path / "p" / "run_counter_collection.csv"),
              ["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value", "Dispatch_Id"], rows)
    bench.summarize_profile(str(tmp_path))
    out = capsys.readouterr().out
    row = [r for r in table_rows(out) if r[0] == "`tree_combine_kernel<8>`"][0]
    # (100 + 300 + 200 + 400) / 2 dispatches = 500; (7 + 9) / 2 = 8
    assert row[1:] == ["1048576", "2", "500", "8"]


def test_summarize_trace_det_atomic(tmp_path, capsys):
    """Kernels are attributed to the roctx range their start falls in; the
    kernel-only time per call is the summed duration over the range's calls."""
    ranges = [("detatom:shrink_1x16x4096_s8:det:2", 0, 1000_000),
              ("detatom:shrink_1x16x4096_s8:atomic:2", 2000_000, 3000_000),
              ("detatom:shrink_1x16x4096_s8:unsplit:2", 4000_000, 5000_000)]
    write_csv(str(tmp_path / "m" / "run_marker_api_trace.csv"),
              ["Function", "Start_Timestamp", "End_Timestamp"],
              [[t, a, b] for t, a, b in ranges])
    kernels = [
        # det: one launch per call, 6 us each
        ["slice_gemm_kernel<Tile<64, 16, 4, 1, 256>, 1, 1, false>(x)", 100_000, 106_000],
        ["slice_gemm_kernel<Tile<64, 16, 4, 1, 256>, 1, 1, false>(x)", 200_000, 206_000],
        # atomic: fill 2 us + slice 4 us per call
        ["fill_zero_kernel(x)", 2100_000, 2102_000],
        ["slice_gemm_kernel<Tile<64, 16, 4, 1, 256>, 1, 2, false>(x)", 2110_000, 2114_000],
        ["fill_zero_kernel(x)", 2200_000, 2202_000],
        ["slice_gemm_kernel<Tile<64, 16, 4, 1, 256>, 1, 2, false>(x)", 2210_000, 2214_000],
        # unsplit: 20 us per call
        ["slice_gemm_kernel<Tile<64, 16, 4, 1, 256>, 1, 0, false>(x)", 4100_000, 4120_000],
        ["slice_gemm_kernel<Tile<64, 16, 4, 1, 256>, 1, 0, false>(x)", 4200_000, 4220_000],
        # outside every range: ignored
        ["fill_zero_kernel(x)", 6000_000, 6900_000],
    ]
    write_csv(str(tmp_path / "k" / "run_kernel_trace.csv"),
              ["Kernel_Name", "Start_Timestamp", "End_Timestamp"], kernels)
    bench.summarize_trace(str(tmp_path))
    row = [r for r in table_rows(capsys.readouterr().out) if r[0] == "shrink_1x16x4096_s8"][0]
    assert row[1:] == ["6.00", "6.00", "20.00", "1.000", "0.300", "1 / 2 / 1"]


def test_write_traffic_calibration(tmp_path, capsys):
    """Each counter is scaled by what it reads for the 256 MiB copy (here the
    copy's FETCH_SIZE reads half its bytes and WRITE_SIZE all of them), only
    the library's kernels are counted, and the sum is per call."""
    mib256_kib = 256 * 1024
    for counter, sub, copy_kib, lib in [("FETCH_SIZE", "fetch", mib256_kib / 2, [(1000, 1), (3000, 2)]),
                                        ("WRITE_SIZE", "write", mib256_kib, [(500, 1), (700, 2)])]:
        rows = [["__amd_rocclr_copyBuffer", counter, copy_kib, 0],
                ["at::native::vectorized_elementwise_kernel", counter, 99999, 9]]
        rows += [["void detred::rmsnorm_kernel<float>(x)", counter, v, d] for v, d in lib]
        write_csv(str(tmp_path / sub / "rmsnorm_b4096" / "run_counter_collection.csv"),
                  ["Kernel_Name", "Counter_Name", "Counter_Value", "Dispatch_Id"], rows)
    bench.write_traffic(str(tmp_path / "fetch"), str(tmp_path / "write"), 2)
    t = json.loads(capsys.readouterr().out)
    assert t["scale_fetch"] == 2.0 and t["scale_write"] == 1.0
    # fetch (1000 + 3000) KiB x 2 + write (500 + 700) KiB x 1, over 2 calls
    assert t["ops"]["rmsnorm_b4096"] == (4000 * 2 + 1200) * 1024 // 2
    assert t["raw_kib_per_call"]["rmsnorm_b4096"] == [2000.0, 600.0]
    assert t["source_hash"] == bench.source_hash()


@pytest.mark.parametrize("current", [True, False])
def test_measured_traffic_only_for_current_sources(tmp_path, monkeypatch, current):
    h = bench.source_hash() if current else "0" * 16
    (tmp_path / "traffic.json").write_text(json.dumps({"source_hash": h,
                                                       "ops": {"dense_m4096": 123456}}))
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.measured_traffic("dense_m4096") == (123456 if current else None)
    assert bench.measured_traffic("not_measured") is None

