"""The benchmark's accounting, on the CPU: algorithmic bytes and flops per
stage against hand-computed values, the bound each workload's dominant call
gets, and the refusal of more than one GPU."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import moe_synth as S  # noqa: E402


def test_stage_work_mixtral_by_hand():
    w = bench.stage_work(S.BY_NAME["mixtral_bf16"])
    T, d, f, k = 4096, 4096, 14336, 2
    A = T * k
    # dispatch: read x once, write k copies, 16 bytes of indices per row
    assert w["dispatch"] == (T * d * 2 + A * d * 2 + 16 * A, 0)
    # expert FFN: 6 d f flops per dispatched row forward, 12 backward
    assert w["grouped_ffn"][1] == 6 * d * f * A == 2_886_218_022_912
    assert w["grouped_ffn_bwd"][1] == 2 * w["grouped_ffn"][1]
    # forward bytes: the 8 experts' W1 and W2 read once, x_perm read, GU
    # [A,2f] saved and O [A,d] written (H stays on chip in the method)
    assert w["grouped_ffn"][0] == 8 * 3 * d * f * 2 + A * d * 2 + A * 2 * f * 2 + A * d * 2
    # combine: k rows per token read, gates and row map, y written
    assert w["combine"] == (A * d * 2 + 8 * A + T * d * 2, 2 * A * d)


def test_stage_work_fp8_payloads():
    d = 7168
    w8 = bench.stage_work(S.BY_NAME["deepseek_v3_fp8"])
    wm = bench.stage_work(S.BY_NAME["deepseek_v3_mxfp8"])
    A = 8192 * 8
    # dispatched row: d codes + fp32 per 128 (FP8) or one byte per 32 (MXFP8)
    assert w8["dispatch"][0] == 8192 * d * 2 + A * (d + 4 * d // 128) + 16 * A
    assert wm["dispatch"][0] == 8192 * d * 2 + A * (d + d // 32) + 16 * A


@pytest.mark.parametrize("name,bound", [("mixtral_bf16", "mfma"), ("qwen3_skew_bf16", "mfma"),
                                        ("deepseek_v3_bf16", "hbm"), ("deepseek_v3_fp8", "hbm"),
                                        ("deepseek_v3_mxfp8", "hbm")])
def test_binding_roofline_of_the_backward_ffn(name, bound):
    cfg = S.BY_NAME[name]
    b, fl = bench.stage_work(cfg)["grouped_ffn_bwd"]
    dt = "fp8" if cfg.weight in ("fp8", "mxfp8") else cfg.act
    t_mfma = fl / (bench.MFMA_PEAK_TFLOPS[dt] * 1e12)
    t_hbm = b / (bench.HBM_PEAK_GBPS * 1e9)
    assert ("mfma" if t_mfma >= t_hbm else "hbm") == bound


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
