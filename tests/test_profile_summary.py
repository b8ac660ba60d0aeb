"""The profile summariser on synthetic rocprofv3 CSVs (CPU): counter values
scaled by the 1 GiB copy's reading, per-launch bytes per GEMM role and per
library call, and the routed / shared split of a step's launches."""
import csv
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

SEL = "void moe::select_kernel<1>(moe::SelArgs)"
G1 = "void moe::gemm_kernel<unsigned short, unsigned short, true, true, 0, 1, 256, 256, 64, 2, 4, 2>(moe::GemmArgs)"
G2 = "void moe::gemm_kernel<unsigned short, unsigned short, true, true, 0, 0, 128, 128, 64, 2, 2, 2>(moe::GemmArgs)"
COPY = "void at::native::copyBuffer_kernel(char*, char const*, long)"


def _write(path, rows, fields):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=fields)
        w.writeheader()
        w.writerows(rows)


def _counters(d, launches):
    rows = [{"Dispatch_Id": i + 1, "Kernel_Name": n, "Counter_Value": v} for i, (n, v) in enumerate(launches)]
    _write(os.path.join(d, "run_counter_collection.csv"), rows, ["Dispatch_Id", "Kernel_Name", "Counter_Value"])


def test_traffic_accounting(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    # two steps, each: select, GEMM1 routed, GEMM1 shared, GEMM2 routed, GEMM2 shared
    seq = [SEL, G1, G1, G2, G2] * 2
    stats = tmp_path / "stats"
    _write(str(stats / "run_kernel_stats.csv"),
           [{"Name": G1, "Calls": 4, "TotalDurationNs": 4000, "AverageNs": 1000},
            {"Name": G2, "Calls": 4, "TotalDurationNs": 2000, "AverageNs": 500},
            {"Name": SEL, "Calls": 2, "TotalDurationNs": 20, "AverageNs": 10}],
           ["Name", "Calls", "TotalDurationNs", "AverageNs"])
    _write(str(stats / "run_kernel_trace.csv"),
           [{"Dispatch_Id": i + 1, "Kernel_Name": n, "Start_Timestamp": 0, "End_Timestamp": 100}
            for i, n in enumerate(seq)],
           ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
    # FETCH_SIZE in KiB: routed GEMM1 1000, shared GEMM1 100, routed GEMM2 500, shared 50
    fetch = {0: 0.0, 1: 1000.0, 2: 100.0, 3: 500.0, 4: 50.0}
    write = {0: 0.0, 1: 10.0, 2: 1.0, 3: 5.0, 4: 0.5}
    _counters(str(tmp_path / "fetch"), [(n, fetch[i % 5]) for i, n in enumerate(seq)])
    _counters(str(tmp_path / "write"), [(n, write[i % 5]) for i, n in enumerate(seq)])
    # the copy moves 1 GiB: FETCH_SIZE reads half of it (factor 2), WRITE_SIZE all (factor 1)
    _counters(str(tmp_path / "cf"), [(COPY, (1 << 30) / 1024 / 2)])
    _counters(str(tmp_path / "cw"), [(COPY, (1 << 30) / 1024)])
    cmd = {k: k for k in ("stats", "fetch", "write", "copy_fetch", "copy_write")}
    bench.summarize_profiles("mixtral_bf16", str(stats), str(tmp_path / "fetch"), str(tmp_path / "write"),
                             str(tmp_path / "cf"), str(tmp_path / "cw"), command=cmd)
    out = json.load(open(tmp_path / "profiles" / "mixtral_bf16_traffic.json"))
    assert out["fetch_factor"] == 2.0 and out["write_factor"] == 1.0
    r = out["roles_bytes_per_launch"]
    assert r["gemm1"] == {"fetch": 1000 * 1024 * 2.0, "write": 10 * 1024 * 1.0}
    assert r["gemm2"] == {"fetch": 500 * 1024 * 2.0, "write": 5 * 1024 * 1.0}
    c = out["calls_bytes_per_launch"]
    assert c["grouped_ffn"] == (1000 + 500) * 1024 * 2.0 + (10 + 5) * 1024
    assert c["shared_ffn"] == (100 + 50) * 1024 * 2.0 + (1 + 0.5) * 1024
    assert out["source_hash"] == bench.source_hash()
    md = open(tmp_path / "profiles" / "mixtral_bf16_kernels.md").read()
    assert "| grouped_ffn |" in md and "| shared_ffn |" in md
