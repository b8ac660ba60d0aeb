"""How much the FP8 layer's weight gradients move when their operands are
quantised too: the measurement behind the FP8 backward reading.

TEST INFRASTRUCTURE ONLY (it calls nothing but ``oracle`` and the seeded
input generators).

The workload definition says only "fp8 e4m3 fwd+bwd". Two readings of the
weight-gradient products dW2 = dO^T H and dW1 = [dG dU]^T X are compared on
the full DeepSeek-V3-style FP8 layer (T = 8192, d = 7168, 256 routed experts
plus one shared, top-8, d_ff = 2048), expert by expert, in fp64:

  unquantised-gradient reading  the forward's dequantised X and H and the
                                unquantised gradients dO, [dG dU]
  token-block reading           all four operands quantised to E4M3 in
                                128-row x 1 blocks inside each expert's rows
                                (fp32 scales amax/448, ragged tail as is)

and both against the unquantised bf16 layer (bf16 weights and inputs taken
exactly, no quantisation anywhere), for context. Prints one JSON line with
the relative L2 errors over all experts (the shared expert included).

With --mx the same comparison on the MXFP8 variant of that layer: every
operand of the forward and data-gradient products in 1 x 32 (activations,
gradients, forward weights) or 32 x 1 (data-gradient weights) E8M0 blocks,
and the token-block reading quantising the four weight-gradient operands in
32-row x 1 E8M0 blocks inside each expert's rows.

    python -m oracle.fp8_wgrad_budget [--experts N] [--mx]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))

import moe_synth as S  # noqa: E402
import oracle  # noqa: E402


def _deq_w(w):
    q, s = oracle.quant_blocks(oracle.as_f32(w), 128, 128)
    return oracle.dequant_blocks(q, s, 128, 128)


def measure(n_experts=None, log=print, mx=False):
    cfg = S.BY_NAME["deepseek_v3_mxfp8" if mx else "deepseek_v3_fp8"]
    x = S.x(cfg)
    dy = oracle.as_f64(S.dy(cfg))
    L, idx, g = oracle.route(cfg, x, S.w_router(cfg))
    counts, offsets, rmap, ptok = oracle.dispatch_index(idx, cfg.E)
    x32 = oracle.as_f32(x)
    # dispatched rows, dequantised
    Xq = oracle.mx_roundtrip_rows(x32) if mx else oracle.fp8_roundtrip_rows(x32)
    X16 = x32.astype(np.float64)                 # the bf16 layer's rows
    # dO of the FP8 layer and of the bf16 layer: gate * dy for every routed row
    gate_of_row = np.empty(cfg.A)
    gate_of_row[rmap.reshape(-1)] = g.reshape(-1)
    tok = ptok
    acc = {k: 0.0 for k in ("g18_r15_1", "g18_r15_2", "r15_1", "r15_2", "r15_ref_1", "r15_ref_2",
                            "g18_ref_1", "g18_ref_2", "ref_1", "ref_2")}
    t0 = time.time()

    def one(Xe, X16e, dOe, w1, w2):
        if mx:
            w1f, w2f = oracle.as_f32(w1), oracle.as_f32(w2)
            W1 = oracle.dequant_mx_rows(*oracle.quant_mx_rows(w1f))
            W2 = oracle.dequant_mx_rows(*oracle.quant_mx_rows(w2f))
            kw = dict(dgrad_quant=oracle.mx_roundtrip_rows,
                      W1d=oracle.dequant_mx_cols(*oracle.quant_mx_cols(w1f)),
                      W2d=oracle.dequant_mx_cols(*oracle.quant_mx_cols(w2f)))
            GU, H, _ = oracle.ffn_fwd(Xe, W1, W2, h_quant=oracle.mx_roundtrip_rows)
            tq = oracle.mx_roundtrip_tokens
        else:
            W1, W2 = _deq_w(w1), _deq_w(w2)
            kw = dict(dgrad_fp8=True)
            GU, H, _ = oracle.ffn_fwd(Xe, W1, W2, h_fp8=True)
            tq = oracle.fp8_roundtrip_tokens
        _, dw1_a, dw2_a, _ = oracle.ffn_bwd(Xe, W1, W2, GU, H, dOe, **kw)
        _, dw1_b, dw2_b, _ = oracle.ffn_bwd(Xe, W1, W2, GU, H, dOe, wgrad_quant=tq, **kw)
        R1, R2 = oracle.as_f64(w1), oracle.as_f64(w2)
        GUr, Hr, _ = oracle.ffn_fwd(X16e, R1, R2)
        _, dw1_r, dw2_r, _ = oracle.ffn_bwd(X16e, R1, R2, GUr, Hr, dOe)
        sq = lambda a: float(np.sum(a * a))
        acc["g18_r15_1"] += sq(dw1_b - dw1_a)
        acc["g18_r15_2"] += sq(dw2_b - dw2_a)
        acc["r15_1"] += sq(dw1_a)
        acc["r15_2"] += sq(dw2_a)
        acc["r15_ref_1"] += sq(dw1_a - dw1_r)
        acc["r15_ref_2"] += sq(dw2_a - dw2_r)
        acc["g18_ref_1"] += sq(dw1_b - dw1_r)
        acc["g18_ref_2"] += sq(dw2_b - dw2_r)
        acc["ref_1"] += sq(dw1_r)
        acc["ref_2"] += sq(dw2_r)

    E = cfg.E if n_experts is None else n_experts
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 > r0:
            rows = tok[r0:r1]
            one(Xq[rows], X16[rows], gate_of_row[r0:r1, None] * dy[rows],
                S.expert_w1(cfg, e), S.expert_w2(cfg, e))
        if e % 16 == 15:
            log(f"[{'mxfp8' if mx else 'fp8'} wgrad] {e + 1} experts, {time.time() - t0:.0f} s")
    one(Xq, X16, dy, S.shared_w1(cfg), S.shared_w2(cfg))   # shared expert: gate 1, every token
    r = lambda a, b: float(np.sqrt(acc[a] / acc[b]))
    return {"workload": cfg.name, "experts": E, "shared": 1,
            "token_block_vs_unquantised_gradient": {"dw1": r("g18_r15_1", "r15_1"),
                                                    "dw2": r("g18_r15_2", "r15_2")},
            "unquantised_gradient_vs_bf16_layer": {"dw1": r("r15_ref_1", "ref_1"),
                                                   "dw2": r("r15_ref_2", "ref_2")},
            "token_block_vs_bf16_layer": {"dw1": r("g18_ref_1", "ref_1"),
                                          "dw2": r("g18_ref_2", "ref_2")},
            "seconds": round(time.time() - t0, 1)}


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--experts", type=int, default=None, help="first N routed experts only")
    ap.add_argument("--mx", action="store_true", help="the MXFP8 variant of the layer")
    a = ap.parse_args()
    print(json.dumps(measure(a.experts, log=lambda m: print(m, file=sys.stderr, flush=True), mx=a.mx)))
