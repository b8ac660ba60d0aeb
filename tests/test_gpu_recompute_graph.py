"""Activation recompute and HIP-graph capture of the whole layer, on the GPU.

Recompute (Megatron Core MoE summary, section 2.2): the backward rebuilds the
SwiGLU output H from the saved gate/up values ("act"), or reruns the first
expert GEMM for both ("full"), instead of keeping them from the forward. The
arithmetic is the same, so every output must equal the saved-activation run
bit for bit; one mode per dtype is also checked against the CPU oracle.

Graph capture (Megatron Core MoE summary, section 2.4: the kernel sequence is
captured once and replayed, and kernels read their dynamic shapes from device
memory): the forward + backward step is captured into one graph; each replay,
after the outputs were scribbled over by eager work, must reproduce the eager
results bit for bit, also after new inputs that route differently were copied
into the captured input buffers.
"""
import numpy as np
import pytest
import torch

import moe_synth as S
import oracle
from test_gpu_parity import SMALL, FORCED_TILE, _check_routing_and_dispatch, _inputs, _np, _say, _tol

pytestmark = pytest.mark.gpu

DEV = "cuda"
OUTPUTS = ("logits", "topk_idx", "topk_gate", "counts", "offsets", "row_id_map", "perm_token",
           "x_perm", "out_perm", "y", "d_gate", "d_out_perm", "dx_perm", "dx", "dw1", "dw2",
           "dw_router")


def _layer(cfg, inp, recompute="none", gemm_tile="auto"):
    from mixture_experts_layer_gather_amd import MoELayer
    layer = MoELayer(**cfg.describe(), recompute=recompute, gemm_tile=gemm_tile, device=DEV)
    cu = lambda t: None if t is None else t.to(DEV)
    layer.set_weights(cu(inp["wr"]), cu(inp["w1"]), cu(inp["w2"]), bias=cu(inp.get("bias")),
                      sw1=cu(inp.get("sw1")), sw2=cu(inp.get("sw2")))
    return layer


def _outputs(layer):
    names = list(OUTPUTS)
    if layer.aux:
        names.append("aux_loss")
    if layer.fp8:
        names.append("x_scale")
    if layer.shared:
        names += ["s_out", "s_dx", "s_dw1", "s_dw2"]
    return {n: getattr(layer, n).clone() for n in names}


def _same(a, b, what):
    for n in a:
        assert torch.equal(a[n], b[n]), f"{what}: {n} differs"


RECOMPUTE_CASES = [("tiny_fp32", "act"), ("tiny_fp32", "full"),
                   ("mixtral_mini", "act"), ("mixtral_mini", "full"),
                   ("qwen_skew_mini_big", "act"), ("qwen_skew_mini_big", "full"),
                   ("deepseek_mini", "act"), ("deepseek_mini", "full"),
                   ("deepseek_fp8_mini", "act"), ("deepseek_fp8_mini", "full"),
                   ("deepseek_mxfp8_mini", "act")]


@pytest.mark.parametrize("name,mode", RECOMPUTE_CASES)
def test_recompute_matches_saved_activations(name, mode):
    cfg = SMALL[name]
    tile = FORCED_TILE.get(name, "auto")
    _say(f"[recompute] {name} mode={mode} tile={tile}")
    inp = _inputs(cfg)
    x, dy = inp["x"].to(DEV), inp["dy"].to(DEV)
    base = _layer(cfg, inp, "none", tile)
    base.step(x, dy)
    rc = _layer(cfg, inp, mode, tile)
    assert rc.act_h is None and (rc.act_gu is None) == (mode == "full")
    rc.step(x, dy)
    torch.cuda.synchronize()
    _same(_outputs(base), _outputs(rc), f"{name} recompute={mode}")


@pytest.mark.parametrize("name", ["tiny_fp32", "mixtral_mini", "deepseek_fp8_mini", "deepseek_mxfp8_mini"])
def test_recompute_against_oracle(name):
    cfg = SMALL[name]
    inp = _inputs(cfg)
    _say(f"[recompute-oracle] {name}")
    layer = _layer(cfg, inp, "act" if cfg.weight == "mxfp8" else "full")
    layer.step(inp["x"].to(DEV), inp["dy"].to(DEV))
    torch.cuda.synchronize()
    ref = oracle.layer(cfg, inp)
    _check_routing_and_dispatch(cfg, layer, ref)
    tol = _tol(cfg)
    for n, got, want in [("y", layer.y, ref["y"]), ("dx", layer.dx, ref["dx"]),
                         ("dw1", layer.dw1, ref["dw1"]), ("dw2", layer.dw2, ref["dw2"]),
                         ("dw_router", layer.dw_router, ref["dw_router"])]:
        err = oracle.rel_l2(_np(got), want)
        assert err <= tol, f"{n}: rel L2 {err:.3e} > {tol}"


def _scribble(layer, outs):
    # eager work between replays: overwrite every output the graph must rewrite
    for n in outs:
        t = getattr(layer, n)
        if t.dtype.is_floating_point:
            t.fill_(float("nan"))
        else:
            t.fill_(-1 if t.dtype != torch.uint8 else 0xAB)


GRAPH_CASES = [("mixtral_mini", "none"), ("qwen_skew_mini", "none"), ("tiny_fp32_aux", "none"),
               ("deepseek_fp8_mini", "none"), ("deepseek_mini_aux", "full"),
               ("mixtral_mini", "act"), ("deepseek_mxfp8_mini", "none")]


@pytest.mark.parametrize("name,mode", GRAPH_CASES)
def test_graph_replay_matches_eager(name, mode):
    cfg = SMALL[name]
    _say(f"[graph] {name} recompute={mode}")
    inp = _inputs(cfg)
    inp2 = dict(inp, x=S.x(cfg.replace(seed_base=cfg.seed_base + 101)),
                dy=S.dy(cfg.replace(seed_base=cfg.seed_base + 101)))
    layer = _layer(cfg, inp, mode)
    x = inp["x"].to(DEV).clone()     # the captured input buffers
    dy = inp["dy"].to(DEV).clone()
    # eager results for both inputs
    layer.step(x, dy)
    torch.cuda.synchronize()
    eager1 = _outputs(layer)
    x2, dy2 = inp2["x"].to(DEV), inp2["dy"].to(DEV)
    layer.step(x2, dy2)
    torch.cuda.synchronize()
    eager2 = _outputs(layer)
    assert not torch.equal(eager1["counts"], eager2["counts"]), "second input should route differently"

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.step(x, dy)   # warm-up on the capture stream's side
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        layer.step(x, dy)
    torch.cuda.synchronize()

    for rep in range(3):
        _scribble(layer, eager1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same(eager1, _outputs(layer), f"{name} replay {rep}")
    # new inputs in the captured buffers: the replay routes them on the device
    x.copy_(x2)
    dy.copy_(dy2)
    for rep in range(2):
        _scribble(layer, eager2)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same(eager2, _outputs(layer), f"{name} replay on new input {rep}")
