"""Host-side pieces of bench.py (no GPU): the HBM traffic summary from two
rocprofv3 counter runs, its staleness check against the kernel sources, and
the kernel-trace table, the refusal of more than one GPU."""
import csv
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as wl  # noqa: E402

WK = "qwen3_4b_L128k_B1024"


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as fh:
        wr = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                            "Counter_Value"])
        wr.writeheader()
        for i, (name, kib) in enumerate(rows):
            wr.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter,
                         "Counter_Value": kib})


def test_traffic_summary_scales_by_the_copy(tmp_path):
    """A counter that reads half of the copy's bytes (FETCH) or all of them
    (WRITE) scales every kernel by 2 and 1; several dispatches of one kernel
    are averaged; kernels missing from either run are left out."""
    w = wl.WORKLOADS[WK]
    copy = w.d * w.d_ff * 4
    f, wr = tmp_path / "fetch.csv", tmp_path / "write.csv"
    _counter_csv(f, "FETCH_SIZE", [
        ("__amd_rocclr_copyBuffer", copy / 2 / 1024),
        ("_ZN5ipttt4mfma8k_gateupINS0_3CfgI", 1000.0),
        ("_ZN5ipttt4mfma8k_gateupINS0_3CfgI", 3000.0),
        ("void ipttt::mfma::k_update<ipttt::mfma::Cfg<1, 2> >(...)", 10.0),
        ("k_conv", 7.0),
    ])
    _counter_csv(wr, "WRITE_SIZE", [
        ("__amd_rocclr_copyBuffer", copy / 1024),
        ("_ZN5ipttt4mfma8k_gateupINS0_3CfgI", 500.0),
        ("void ipttt::mfma::k_update<ipttt::mfma::Cfg<1, 2> >(...)", 20.0),
    ])
    t = bench.summarize_traffic(WK, str(f), str(wr))
    assert t["calibration"] == {"copy_bytes": copy, "fetch_factor": 2.0, "write_factor": 1.0}
    b = t["bytes_per_launch"]
    assert set(b) == {"gateup", "update"}  # conv has no WRITE_SIZE row
    assert b["gateup"] == {"fetch": 2 * 2000 * 1024, "write": 500 * 1024,
                           "total": 2 * 2000 * 1024 + 500 * 1024}
    assert b["update"] == {"fetch": 2 * 10 * 1024, "write": 20 * 1024,
                           "total": 2 * 10 * 1024 + 20 * 1024}
    assert t["kernel_source_sha"] == bench.kernel_source_hash()


def test_traffic_is_null_once_the_kernels_change(tmp_path, monkeypatch):
    path = tmp_path / f"traffic_{WK}.json"
    monkeypatch.setattr(bench, "traffic_path", lambda workload: str(path))
    assert bench.load_traffic(WK, "gateup") is None  # no summary
    rec = {"workload": WK, "kernel_source_sha": bench.kernel_source_hash(),
           "bytes_per_launch": {"gateup": {"fetch": 3, "write": 4, "total": 7}}}
    path.write_text(json.dumps(rec))
    assert bench.load_traffic(WK, "gateup") == 7
    assert bench.load_traffic(WK, "apply") is None  # kernel not measured
    rec["kernel_source_sha"] = "0" * 16
    path.write_text(json.dumps(rec))
    assert bench.load_traffic(WK, "gateup") is None  # stale


def test_kernel_source_hash_covers_the_kernel_sources(tmp_path, monkeypatch):
    a, b = tmp_path / "a.hip", tmp_path / "b.h"
    a.write_text("x")
    b.write_text("y")
    monkeypatch.setattr(bench, "KERNEL_SRCS", [str(a), str(b)])
    h0 = bench.kernel_source_hash()
    b.write_text("y ")
    assert bench.kernel_source_hash() != h0


def test_trace_summary_names_and_order(tmp_path):
    p = tmp_path / "stats.csv"
    with open(p, "w", newline="") as fh:
        wr = csv.DictWriter(fh, fieldnames=["Name", "Calls", "TotalDurationNs", "AverageNs",
                                            "MinNs", "MaxNs", "Percentage"])
        wr.writeheader()
        wr.writerow({"Name": "__amd_rocclr_copyBuffer", "Calls": 3, "TotalDurationNs": 120000,
                     "AverageNs": 40000, "MinNs": 36000, "MaxNs": 41000, "Percentage": 0.1})
        wr.writerow({"Name": "_ZN5ipttt4mfma8k_gateupINS0_3CfgILi2ELi4EEELb1EEEvNS_4SlabE",
                     "Calls": 3, "TotalDurationNs": 30000000, "AverageNs": 10000000,
                     "MinNs": 9900000, "MaxNs": 10100000, "Percentage": 60.0})
        wr.writerow({"Name": "void ipttt::mfma::k_update<ipttt::mfma::Cfg<1, 2> >(ipttt::Slab)",
                     "Calls": 3, "TotalDurationNs": 24000000, "AverageNs": 8000000,
                     "MinNs": 7900000, "MaxNs": 8100000, "Percentage": 39.9})
    lines = bench.trace_summary(str(p)).splitlines()
    assert lines[2] == "| `k_gateup` | 3 | 10.000 | 9.900 | 10.100 | 60.00 |"
    assert lines[3] == "| `k_update<Cfg<1, 2> >` | 3 | 8.000 | 7.900 | 8.100 | 39.90 |"
    assert lines[4].startswith("| `copyBuffer` | 3 | 0.040 |")


def test_more_than_one_gpu_is_refused():
    """The library runs on one GPU: --gpus above 1 prints a JSON error line and
    exits with status 2 before touching a device."""
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_step_stats_median_min_max():
    assert bench.step_stats([3.0, 1.0, 2.0]) == {"median": 2.0, "min": 1.0, "max": 3.0}
    assert bench.step_stats([4.0, 1.0, 2.0, 3.0]) == {"median": 2.5, "min": 1.0, "max": 4.0}
    assert bench.step_stats([5.0]) == {"median": 5.0, "min": 5.0, "max": 5.0}
