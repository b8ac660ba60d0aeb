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


LOG = "void moe::logits_small_e_kernel<unsigned short, 8>(unsigned short const*, float const*, float const*, float*, int, int, int)"
CNT = "moe::dispatch_count_kernel(int const*, int*, int, int, int)"
POS = "void moe::dispatch_pos_kernel<true>(int const*, int const*, int*, int*, int*, int*, int, int, int)"
GAT = "void moe::dispatch_gather_kernel<unsigned short>(unsigned short const*, int const*, unsigned short*, int, int, int)"
COMB = "void moe::combine_kernel<unsigned short, 2>(unsigned short const*, int const*, float const*, unsigned short const*, unsigned short*, int, int, int)"
CBWD = "void moe::combine_bwd_kernel<unsigned short, 2>(unsigned short const*, unsigned short const*, int const*, float const*, unsigned short*, float*, int, int, int)"
DH = "void moe::gemm_kernel<unsigned short, unsigned short, true, false, 0, 2, 256, 256, 64, 2, 4, 2>(moe::GemmArgs)"
DX = "void moe::gemm_kernel<unsigned short, unsigned short, true, false, 0, 0, 128, 128, 64, 2, 2, 2>(moe::GemmArgs)"
WG = "void moe::gemm_kernel<unsigned short, unsigned short, false, false, 1, 0, 128, 256, 32, 2, 2, 3>(moe::GemmArgs)"
DL = "void moe::dlogits_kernel<1>(moe::DLArgs)"
RG = "void moe::rgemm_bf16_kernel<unsigned short, false, float, 0>(moe::VArgs)"
FILL = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<unsigned char>, std::array<char*, 1ul> >(int, at::native::FillFunctor<unsigned char>, std::array<char*, 1ul>)"
QT = "void moe::quant_tiles128_kernel<unsigned short>(unsigned short const*, unsigned char*, float*, long, int)"

# one step of the Mixtral-style layer, call by call; the flush (a torch
# fill) between steps and a set-up kernel before the first step are not
# the library's
STEP = [("route", LOG), ("route", SEL), ("dispatch", CNT), ("dispatch", POS), ("dispatch", GAT),
        ("grouped_ffn", G1), ("grouped_ffn", G2), ("combine", COMB), ("combine_bwd", CBWD),
        ("grouped_ffn_bwd", DH), ("grouped_ffn_bwd", DX), ("grouped_ffn_bwd", WG),
        ("grouped_ffn_bwd", WG), ("dispatch_bwd", COMB), ("route_bwd", DL), ("route_bwd", RG),
        ("route_bwd", RG)]


def test_call_attribution():
    import moe_synth as S
    seq = [QT] + [n for _, n in STEP] + [FILL] + [n for _, n in STEP]
    rows = [{"Dispatch_Id": i + 1, "Kernel_Name": n} for i, n in enumerate(seq)]
    att = bench.attribute_calls(rows, bench.step_calls(S.BY_NAME["mixtral_bf16"]))
    assert [(s, c, r["Kernel_Name"]) for s, c, r in att] == \
        [(0, c, n) for c, n in STEP] + [(1, c, n) for c, n in STEP]


def test_traffic_accounting(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    seq = [QT] + ([n for _, n in STEP] + [FILL]) * 2
    calls = [None] + ([c for c, _ in STEP] + [None]) * 2
    stats = tmp_path / "stats"
    _write(str(stats / "run_kernel_stats.csv"),
           [{"Name": n, "Calls": 2, "TotalDurationNs": 200, "AverageNs": 100} for n in sorted(set(seq))],
           ["Name", "Calls", "TotalDurationNs", "AverageNs"])
    # durations: 1000 ns for each GEMM launch, 10 for every other kernel
    dur = lambda n: 1000 if "gemm_kernel" in n else 10
    _write(str(stats / "run_kernel_trace.csv"),
           [{"Dispatch_Id": i + 1, "Kernel_Name": n, "Start_Timestamp": 0, "End_Timestamp": dur(n)}
            for i, n in enumerate(seq)],
           ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
    # FETCH_SIZE in KiB: 1000 per GEMM launch, 1 per other kernel; WRITE_SIZE a tenth
    _counters(str(tmp_path / "fetch"), [(n, 1000.0 if "gemm" in n else 1.0) for n in seq])
    _counters(str(tmp_path / "write"), [(n, 100.0 if "gemm" in n else 0.1) for n in seq])
    # the copy moves 1 GiB: FETCH_SIZE reads half of it (factor 2), WRITE_SIZE all (factor 1)
    _counters(str(tmp_path / "cf"), [(COPY, (1 << 30) / 1024 / 2)])
    _counters(str(tmp_path / "cw"), [(COPY, (1 << 30) / 1024)])
    cmd = {k: k for k in ("stats", "fetch", "write", "copy_fetch", "copy_write")}
    bench.summarize_profiles("mixtral_bf16", str(stats), str(tmp_path / "fetch"), str(tmp_path / "write"),
                             str(tmp_path / "cf"), str(tmp_path / "cw"), command=cmd)
    out = json.load(open(tmp_path / "profiles" / "mixtral_bf16_traffic.json"))
    assert out["fetch_factor"] == 2.0 and out["write_factor"] == 1.0
    r = out["roles_bytes_per_launch"]
    assert r["gemm1"] == {"fetch": 1000 * 1024 * 2.0, "write": 100 * 1024 * 1.0}
    assert r["wgrad"] == r["dx"] == r["gemm2"]
    c = out["calls_bytes_per_launch"]
    assert c["grouped_ffn_bwd"] == 4 * (1000 * 1024 * 2.0 + 100 * 1024)
    assert abs(c["dispatch"] - 3 * (1024 * 2.0 + 0.1 * 1024)) < 1e-6
    assert "shared_ffn" not in c
    ms = out["calls_ms_per_step"]
    assert ms["grouped_ffn_bwd"] == 4000 / 1e6 and ms["route_bwd"] == 30 / 1e6
    assert out["source_hash"] == bench.source_hash()
    md = open(tmp_path / "profiles" / "mixtral_bf16_kernels.md").read()
    assert "| grouped_ffn |" in md and "| grouped_ffn_bwd | 0.004 |" in md
