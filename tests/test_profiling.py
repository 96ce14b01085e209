"""The rocprofv3 summary tool on small synthetic trace and counter files:
dispatch windows, grid split, percentiles and the calibration-copy scale."""
import csv
import os

import pytest

from compressed_gemv_amd import profiling as pf


def _write(path, fields, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        w.writerows(rows)


def _trace(d):
    fields = ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"]
    rows, t = [], 1000
    # 5 dispatches of kernel A at grid 64 (1..5 us), then 3 of A at grid 128 (10 us), then B
    for i in range(5):
        rows.append({"Kernel_Name": "void ns::A<4, 64>(int const*)", "Start_Timestamp": t,
                     "End_Timestamp": t + 1000 * (i + 1), "Grid_Size_X": 64, "Grid_Size_Y": 1, "Grid_Size_Z": 1})
        t += 100000
    for _ in range(3):
        rows.append({"Kernel_Name": "void ns::A<4, 64>(int const*)", "Start_Timestamp": t,
                     "End_Timestamp": t + 10000, "Grid_Size_X": 128, "Grid_Size_Y": 1, "Grid_Size_Z": 1})
        t += 100000
    rows.append({"Kernel_Name": "B(float)", "Start_Timestamp": t, "End_Timestamp": t + 2000,
                 "Grid_Size_X": 1, "Grid_Size_Y": 1, "Grid_Size_Z": 1})
    _write(os.path.join(d, "x", "run_kernel_trace.csv"), fields, rows[::-1])   # file order != time order


def _counters(d, kib_a, kib_copy):
    fields = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]
    rows = [{"Dispatch_Id": i, "Kernel_Name": "void ns::A<4, 64>(int const*)", "Grid_Size": 64,
             "Counter_Name": "C", "Counter_Value": kib_a + i} for i in range(5)]
    rows.append({"Dispatch_Id": 9, "Kernel_Name": "__amd_rocclr_copyBuffer", "Grid_Size": 1, "Counter_Name": "C",
                 "Counter_Value": kib_copy})
    _write(os.path.join(d, "y", "run_counter_collection.csv"), fields, rows)


def test_groups_and_windows(tmp_path):
    _trace(str(tmp_path / "t"))
    g = pf.dispatch_groups(str(tmp_path / "t"))
    assert g[("void ns::A<4, 64>", "64")] == [1.0, 2.0, 3.0, 4.0, 5.0]
    assert g[("void ns::A<4, 64>", "128")] == [10.0] * 3
    assert g[("B", "1")] == [2.0]
    d = pf.dist([5.0, 1.0, 2.0, 3.0, 4.0, 6.0, 7.0, 8.0, 9.0, 10.0])
    assert (d["median"], d["p10"], d["p90"], d["min"], d["max"]) == (5.5, 2.0, 9.0, 1.0, 10.0)
    s = pf.summarize(str(tmp_path / "t"), None, None, "A<4, 64>", 4e6, skip=1, take=3, grid="64")
    assert s["duration_us"]["n"] == 3 and s["duration_us"]["mean"] == pytest.approx(3.0)
    assert s["achieved_gbs"] == pytest.approx(4e6 / 3e-6 / 1e9)


def test_traffic_scale(tmp_path):
    _trace(str(tmp_path / "t"))
    _counters(str(tmp_path / "f"), 1000.0, 524288.0)     # the copy's 1 GiB reads as 512 MiB: scale 2
    _counters(str(tmp_path / "w"), 10.0, 1048576.0)      # writes read 1:1
    s = pf.summarize(str(tmp_path / "t"), str(tmp_path / "f"), str(tmp_path / "w"), "A<4, 64>", 4e6,
                     skip=1, take=3, grid="64")
    assert s["fetch_scale"] == pytest.approx(2.0) and s["write_scale"] == pytest.approx(1.0)
    # dispatches 1..3 -> fetch 1001..1003 KiB (median 1002), write 11..13 (median 12)
    assert s["traffic_bytes"] == pytest.approx(1002 * 1024 * 2 + 12 * 1024)


def test_kernel_spec():
    assert pf._kernel_spec("gemv_b1_kernel<4, 64=132120576@1024+25:20") == (
        "gemv_b1_kernel<4, 64", 132120576.0, "1024", 25, 20)
    assert pf._kernel_spec("bin_mfma_kernel<2=100") == ("bin_mfma_kernel<2", 100.0, None, 0, 0)


def test_counter_table(tmp_path):
    _counters(str(tmp_path / "c"), 100.0, 1.0)
    t = pf.counter_table([str(tmp_path / "c")], "A<4, 64>", grid="64", skip=1, take=3)
    assert t == {"C": 102.0}
