"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Integer and index outputs (logits under the fixed fp32 order, top-k indices,
counts, offsets, row map, token permutation, dispatched rows) are compared bit
for bit; floating-point outputs by relative L2 error against the fp64 oracle
with the tolerance of their precision: 1e-5 (fp32), 2e-2 (bf16), 6e-2 (fp8).
Small layers and full-size layers are compared on every element; at full
size the oracle runs expert by expert and the comparison accumulates each
tensor's error piece by piece.
"""
import os
import sys

import numpy as np
import pytest
import torch

import moe_synth as S
import oracle

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 6e-2}
DEV = "cuda"


_CAPMAN = None


@pytest.fixture(autouse=True)
def _progress_to_terminal(request):
    """Lets _say reach the terminal while pytest captures output: the full-
    size tests run their CPU oracle for minutes, and a run that prints
    nothing for that long looks hung."""
    global _CAPMAN
    _CAPMAN = request.config.pluginmanager.getplugin("capturemanager")
    yield
    _CAPMAN = None


def _say(msg):
    if _CAPMAN is not None:
        with _CAPMAN.global_and_fixture_disabled():
            print(msg, flush=True)
    else:
        print(msg, flush=True)
    sys.stdout.flush()


def _tol(cfg):
    return TOL["fp8"] if cfg.weight in ("fp8", "mxfp8") else TOL[cfg.act]


def _np(t):
    if t.dtype in (torch.int32, torch.int64, torch.uint8):
        return t.cpu().numpy()
    return t.float().cpu().numpy()


def _inputs(cfg, threads=8):
    w1, w2 = S.all_expert_weights(cfg, threads=threads)
    inp = dict(x=S.x(cfg), wr=S.w_router(cfg), bias=S.router_bias(cfg), w1=w1, w2=w2,
               dy=S.dy(cfg))
    if cfg.shared:
        inp.update(sw1=S.shared_w1(cfg), sw2=S.shared_w2(cfg))
    return inp


def _gpu_layer(cfg, inp, identity=False, gemm_tile="auto"):
    from mixture_experts_layer_gather_amd import MoELayer
    layer = MoELayer(**cfg.describe(), identity=identity, gemm_tile=gemm_tile, device=DEV)
    cu = lambda t: None if t is None else t.to(DEV)
    layer.set_weights(cu(inp["wr"]), cu(inp["w1"]), cu(inp["w2"]), bias=cu(inp.get("bias")),
                      sw1=cu(inp.get("sw1")), sw2=cu(inp.get("sw2")))
    layer.step(cu(inp["x"]), cu(inp["dy"]))
    torch.cuda.synchronize()
    return layer


def _check_routing_and_dispatch(cfg, layer, ref):
    assert np.array_equal(_np(layer.logits), ref["logits"]), "logits not bit-exact"
    assert np.array_equal(_np(layer.topk_idx), ref["idx"]), "top-k indices differ"
    for name in ("counts", "offsets", "row_id_map", "perm_token"):
        assert np.array_equal(_np(getattr(layer, name)), ref[name]), name
    rm = _np(layer.routing_map)
    exp = np.zeros((cfg.T, cfg.E), np.uint8)
    np.put_along_axis(exp, ref["idx"].astype(np.int64), 1, axis=1)
    assert np.array_equal(rm, exp), "routing map"
    assert oracle.rel_l2(_np(layer.topk_gate), ref["gates"]) <= 1e-6, "gates"


def _compare_small(cfg, identity=False, inp=None, gemm_tile="auto"):
    inp = inp or _inputs(cfg)
    _say(f"[parity] {cfg.name} T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} f={cfg.f} id={identity} "
         f"tile={gemm_tile}")
    layer = _gpu_layer(cfg, inp, identity, gemm_tile)
    ref = oracle.layer(cfg, inp, identity=identity)
    _check_routing_and_dispatch(cfg, layer, ref)
    if cfg.weight in ("fp8", "mxfp8"):
        assert np.array_equal(_np(layer.x_perm), ref["xq_perm"]), "fp8 dispatch codes"
        assert np.array_equal(_np(layer.x_scale), ref["x_scale_perm"]), "fp8 dispatch scales"
    else:
        assert np.array_equal(_np(layer.x_perm), ref["x_perm"]), "x_perm"
    tol = _tol(cfg)
    if cfg.aux_coeff:
        err = abs(float(layer.aux_loss.item()) - ref["aux_loss"]) / ref["aux_loss"]
        assert err <= 1e-5, f"aux_loss rel {err:.2e}"
    pairs = [("y", layer.y, ref["y"]), ("d_gate", layer.d_gate, ref["d_gate"]),
             ("dx", layer.dx, ref["dx"])]
    if identity and cfg.renorm:
        # every slot then sees the same d_gate, so the exact router gradient
        # is zero: bound the GPU's against the scale of its factors instead
        scale = np.linalg.norm(ref["d_gate"]) * np.linalg.norm(oracle.as_f64(inp["x"]))
        assert np.linalg.norm(_np(layer.dw_router)) <= 1e-5 * scale
    else:
        pairs.append(("dw_router", layer.dw_router, ref["dw_router"]))
    if not identity:
        pairs += [("out_perm", layer.out_perm, ref["out_perm"]),
                  ("dw1", layer.dw1, ref["dw1"]), ("dw2", layer.dw2, ref["dw2"])]
        if cfg.shared:
            pairs += [("shared_dw1", layer.s_dw1[0], ref["shared_dw1"]),
                      ("shared_dw2", layer.s_dw2[0], ref["shared_dw2"])]
    for name, got, want in pairs:
        err = oracle.rel_l2(_np(got), want)
        assert err <= tol, f"{name}: rel L2 {err:.3e} > {tol}"
    if not identity:
        # experts that received no rows must get exact zero gradients
        empty = np.nonzero(ref["counts"] == 0)[0]
        if empty.size:
            assert not _np(layer.dw1[torch.as_tensor(empty)]).any()
            assert not _np(layer.dw2[torch.as_tensor(empty)]).any()
    return layer, ref


# ------------------------------------------------------------ small layers

SMALL = {
    "tiny_fp32": S.BY_NAME["tiny_fp32"],
    "mixtral_mini": S.mini(S.BY_NAME["mixtral_bf16"], T=1000, d=256, f=384),
    # >= 512 rows per expert and 256-multiple widths, run with the 256 x 256
    # tile forced on every GEMM (too few tiles for the shape-based choice)
    "mixtral_mini_bigtile": S.mini(S.BY_NAME["mixtral_bf16"], T=2304, d=512, f=512, seed_base=33),
    "mixtral_mini_f32": S.mini(S.BY_NAME["mixtral_bf16"], T=333, d=128, f=256).replace(act="f32", weight="f32"),
    "deepseek_mini": S.mini(S.BY_NAME["deepseek_v3_bf16"], T=300, d=256, f=256, E=32).replace(k=6),
    "qwen_skew_mini": S.mini(S.BY_NAME["qwen3_skew_bf16"], T=700, d=256, f=128, E=16).replace(k=4),
    # 256 x 256 tiles forced where the widths allow (GEMM1, GEMM2 and dX; f =
    # 128 keeps dH and the weight gradients on 128 x 128): mixed tile sizes
    # and ragged groups smaller than a tile
    "qwen_skew_mini_big": S.mini(S.BY_NAME["qwen3_skew_bf16"], T=700, d=256, f=128, E=16).replace(k=4, seed_base=34),
    "deepseek_fp8_mini": S.mini(S.BY_NAME["deepseek_v3_fp8"], T=400, d=384, f=256, E=32).replace(k=6),
    # FP8 with the 256 x 256 tile forced on all four row-grouped products
    # (d and 2f multiples of 256), ragged experts of 0 to a few hundred rows
    "deepseek_fp8_mini_big": S.mini(S.BY_NAME["deepseek_v3_fp8"], T=600, d=512, f=256, E=16).replace(
        k=4, num_groups=4, topk_groups=2, seed_base=35),
    # FP8 weight gradients in runs of two column tiles per workgroup (64
    # experts x 8 x 9 tiles of dW1), the last run of each row block one tile
    # short. Even routing: experts of one 128-row block, so each tile's only
    # K step ends it and two tiles' stores sit between a load and its wait;
    # skewed routing: experts of one block, of several, and with no rows
    "deepseek_fp8_runs": S.mini(S.BY_NAME["deepseek_v3_fp8"], T=1024, d=1152, f=512, E=64).replace(k=4, seed_base=36),
    "deepseek_fp8_runs_skew": S.mini(S.BY_NAME["deepseek_v3_fp8"], T=1024, d=1152, f=512, E=64).replace(
        k=4, bias="zipf", seed_base=37),
    # bf16 weight gradients of short experts (persistent runs of two
    # 128 x 128 column tiles, the last run of each row block one tile short):
    # even routing, and skewed routing with empty and multi-block experts
    "deepseek_bf16_runs": S.mini(S.BY_NAME["deepseek_v3_bf16"], T=1024, d=1152, f=512, E=64).replace(k=4, seed_base=44),
    "deepseek_bf16_runs_skew": S.mini(S.BY_NAME["deepseek_v3_bf16"], T=1024, d=1152, f=512, E=64).replace(
        k=4, bias="zipf", seed_base=45),
    # 8-bit layers whose experts average 256 rows (more than 128, at most
    # 320): the 160 x 128 tile; even and skewed routing (experts of one to
    # several row tiles, empty experts), FP8 and MXFP8
    "deepseek_fp8_mid": S.mini(S.BY_NAME["deepseek_v3_fp8"], T=1024, d=384, f=256, E=16).replace(
        k=4, num_groups=4, topk_groups=2, seed_base=46),
    "deepseek_fp8_mid_skew": S.mini(S.BY_NAME["deepseek_v3_fp8"], T=1024, d=384, f=256, E=16).replace(
        k=4, num_groups=4, topk_groups=2, bias="zipf", seed_base=47),
    "deepseek_mxfp8_mid": S.mini(S.BY_NAME["deepseek_v3_mxfp8"], T=1024, d=384, f=256, E=16).replace(
        k=4, num_groups=4, topk_groups=2, seed_base=48),
    # the other group rule (a group's best score instead of its best two)
    # and sigmoid gates without renormalisation
    "deepseek_mini_gmax": S.mini(S.BY_NAME["deepseek_v3_bf16"], T=300, d=256, f=256, E=32).replace(
        k=6, group_score="max", seed_base=61),
    "deepseek_mini_norenorm": S.mini(S.BY_NAME["deepseek_v3_bf16"], T=300, d=256, f=256, E=32).replace(
        k=6, renorm=False, gate_scale=1.0, seed_base=62),
    # the largest expert count and top-k the library takes (E = 1024,
    # k = 16): most experts get 0 to 3 rows
    "max_experts_topk": S.mini(S.BY_NAME["mixtral_bf16"], T=200, d=128, f=128, E=1024).replace(k=16, seed_base=63),
    # MXFP8: 1 x 32 / 32 x 1 blocks with E8M0 scales on the matrix cores
    "deepseek_mxfp8_mini": S.mini(S.BY_NAME["deepseek_v3_mxfp8"], T=400, d=384, f=256, E=32).replace(k=6),
    # MXFP8 weight gradients (32-row E8M0 token blocks) in runs of two column
    # tiles, as for FP8 above: even routing, and skewed routing with empty
    # experts and experts whose last 128-row block ends inside a 32-row block
    "deepseek_mxfp8_runs": S.mini(S.BY_NAME["deepseek_v3_mxfp8"], T=1024, d=1152, f=512, E=64).replace(
        k=4, seed_base=38),
    "deepseek_mxfp8_runs_skew": S.mini(S.BY_NAME["deepseek_v3_mxfp8"], T=1024, d=1152, f=512, E=64).replace(
        k=4, bias="zipf", seed_base=39),
    # the load-balancing auxiliary loss on (coefficient 0.01): its value and
    # its share of the router gradient
    "mixtral_mini_aux": S.mini(S.BY_NAME["mixtral_bf16"], T=1000, d=256, f=384).replace(aux_coeff=0.01),
    "tiny_fp32_aux": S.BY_NAME["tiny_fp32"].replace(aux_coeff=0.01),
    "deepseek_mini_aux": S.mini(S.BY_NAME["deepseek_v3_bf16"], T=300, d=256, f=256, E=32).replace(
        k=6, aux_coeff=0.01),
}


FORCED_TILE = {"mixtral_mini_bigtile": "big", "qwen_skew_mini_big": "big", "deepseek_fp8_mini_big": "big"}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_layer_parity(name):
    _compare_small(SMALL[name], gemm_tile=FORCED_TILE.get(name, "auto"))


def test_forced_small_tiles():
    # the 128 x 128 tile on shapes that would take the 256 x 256 one
    _compare_small(SMALL["mixtral_mini_bigtile"], gemm_tile="small")


@pytest.mark.parametrize("name", ["tiny_fp32", "deepseek_mini"])
def test_identity_experts(name):
    cfg = SMALL[name]
    layer, ref = _compare_small(cfg, identity=True)
    x = oracle.as_f64(S.x(cfg))
    g = ref["gates"].sum(1, keepdims=True) + (1.0 if cfg.shared else 0.0)
    assert oracle.rel_l2(_np(layer.y), g * x) <= _tol(cfg)


def test_edge_shapes():
    base = S.mini(S.BY_NAME["mixtral_bf16"], T=1, d=128, f=128, E=8)
    for cfg in [base,                                    # a single token
                base.replace(T=37, k=4, E=4, seed_base=40),    # k = E
                base.replace(T=50, k=1, E=1, seed_base=41),    # one expert
                base.replace(T=257, seed_base=42),             # chunk tail
                base.replace(T=64, act="f32", weight="f32", k=3, seed_base=43)]:
        _compare_small(cfg)


@pytest.mark.parametrize("name", ["tiny_fp32", "mixtral_mini", "deepseek_fp8_mini", "deepseek_mxfp8_mini"])
def test_empty_batch(name):
    """T = 0: no rows for any expert, so counts, offsets and every weight
    gradient are exact zeros (and the auxiliary loss is 0); the T-row
    outputs are empty. The outputs are filled with garbage first."""
    from mixture_experts_layer_gather_amd import MoELayer
    cfg = SMALL[name].replace(T=0, aux_coeff=0.01)
    _say(f"[empty] {name}")
    inp = _inputs(cfg)
    layer = MoELayer(**cfg.describe(), device=DEV)
    cu = lambda t: None if t is None else t.to(DEV)
    layer.set_weights(cu(inp["wr"]), cu(inp["w1"]), cu(inp["w2"]), bias=cu(inp.get("bias")),
                      sw1=cu(inp.get("sw1")), sw2=cu(inp.get("sw2")))
    outs = ["counts", "offsets", "dw1", "dw2", "dw_router", "aux_loss"]
    if cfg.shared:
        outs += ["s_dw1", "s_dw2"]
    for n in outs:
        t = getattr(layer, n)
        t.fill_(float("nan") if t.dtype.is_floating_point else -7)
    layer.step(cu(inp["x"]), cu(inp["dy"]))
    torch.cuda.synchronize()
    for n in outs:
        assert not _np(getattr(layer, n)).any(), n
    assert layer.y.shape == (0, cfg.d) and layer.dx.shape == (0, cfg.d)


def test_all_equal_logits_pick_lowest_indices():
    cfg = S.mini(S.BY_NAME["mixtral_bf16"], T=100, d=128, f=128, E=8).replace(k=3)
    inp = _inputs(cfg)
    inp["wr"] = torch.zeros_like(inp["wr"])
    layer, ref = _compare_small(cfg, inp=inp)
    assert np.array_equal(_np(layer.topk_idx), np.tile(np.arange(3), (100, 1)))


def test_deterministic_repeat():
    cfg = SMALL["qwen_skew_mini"]
    inp = _inputs(cfg)
    a = _gpu_layer(cfg, inp)
    outs = {n: _np(getattr(a, n)).copy() for n in ("y", "dx", "dw1", "dw2", "dw_router", "d_gate")}
    b = _gpu_layer(cfg, inp)
    for n, v in outs.items():
        assert np.array_equal(v, _np(getattr(b, n))), n


# ------------------------------------------------------------ fp8 pieces

def test_fp8_block_quantiser_bit_exact():
    from mixture_experts_layer_gather_amd import moe_quantize_fp8_blockwise
    g = torch.Generator().manual_seed(11)
    # whole 128 x 128 blocks (register path) and ragged edges (general path)
    for R, C in [(384, 640), (300, 520)]:
        src = torch.randn(R, C, generator=g) * torch.exp(torch.randn(R, 1, generator=g) * 3)
        src[7, :128] = 0.0
        src[9, 5] = 1e30
        src[200:256, 128:256] = 0.0  # an all-zero 128 x 128 block: scale 1, codes 0
        for br, bc in [(128, 128), (1, 128)]:
            for dt in (torch.float32, torch.bfloat16):
                s = src.to(dt)
                q = torch.empty(R, C, dtype=torch.uint8, device=DEV)
                sc = torch.empty(-(-R // br), -(-C // bc), dtype=torch.float32, device=DEV)
                moe_quantize_fp8_blockwise(s.to(DEV), R, C, br, bc, q, sc)
                torch.cuda.synchronize()
                rq, rs = oracle.quant_blocks(oracle.as_f32(s), br, bc)
                assert np.array_equal(_np(sc), rs), (R, C, br, bc, dt)
                assert np.array_equal(_np(q), rq), (R, C, br, bc, dt)


def test_fp8_encoder_exhaustive_in_range():
    """Every fp32 value with |v| <= 448 quantised with scale 1 (a 1 x 2^k
    block holding 448 fixes the scale to exactly 1)."""
    from mixture_experts_layer_gather_amd import moe_quantize_fp8_blockwise
    top = int(np.array(448.0, np.float32).view(np.uint32))
    step = 1 << 24
    for sign in (0, 1 << 31):
        for lo in range(0, top + 1, step):
            hi = min(lo + step, top + 1)
            bits = (np.arange(lo, hi, dtype=np.uint64) | sign).astype(np.uint32)
            v = bits.view(np.float32).copy()
            n = v.size
            cols = 1 << 20
            pad = (-n) % cols
            v = np.concatenate([v, np.zeros(pad, np.float32)]).reshape(-1, cols)
            v[:, 0] = 448.0 if sign == 0 else -448.0   # pins amax, scale = 1
            src = torch.from_numpy(v).to(DEV)
            q = torch.empty(v.shape, dtype=torch.uint8, device=DEV)
            sc = torch.empty(v.shape[0], 1, dtype=torch.float32, device=DEV)
            moe_quantize_fp8_blockwise(src, v.shape[0], cols, 1, cols, q, sc)
            torch.cuda.synchronize()
            assert np.all(_np(sc) == 1.0)
            assert np.array_equal(_np(q), oracle.e4m3_encode(v)), hex(lo | sign)


def test_mxfp8_quantiser_bit_exact():
    """moe_quantize_mxfp8 in both block orientations against the oracle:
    codes and E8M0 bytes bit for bit, over blocks whose magnitudes span the
    fp32 range (zero blocks, lone subnormals, values at powers of two)."""
    from mixture_experts_layer_gather_amd import moe_quantize_mxfp8
    g = torch.Generator().manual_seed(12)
    R, C = 256, 640
    src = torch.randn(R, C, generator=g) * torch.exp(torch.randn(R, 1, generator=g) * 12)
    src[:, 5] *= torch.exp(torch.randn(R, generator=g) * 20)     # one outlier column
    src[3, :32] = 0.0
    src[:32, 100] = 0.0
    src[4, 32:64] = 0.0
    src[4, 40] = -2.0e-40                                        # an fp32 subnormal alone
    src[5, :32] = torch.tensor([2.0 ** i for i in range(-16, 16)])
    src[6, :] = 448.0 * 2.0 ** 30
    for dt in (torch.float32, torch.bfloat16):
        s = src.to(dt)
        s32 = s.float().numpy()
        for colwise in (False, True):
            q = torch.empty(R, C, dtype=torch.uint8, device=DEV)
            e = torch.empty((R // 32, C) if colwise else (R, C // 32), dtype=torch.uint8, device=DEV)
            moe_quantize_mxfp8(s.to(DEV), R, C, colwise, q, e)
            torch.cuda.synchronize()
            rq, re = (oracle.quant_mx_cols if colwise else oracle.quant_mx_rows)(s32)
            assert np.array_equal(_np(e), re), (dt, colwise, "scales")
            assert np.array_equal(_np(q), rq), (dt, colwise, "codes")


def test_fp8_dispatch_bit_exact():
    from mixture_experts_layer_gather_amd import make_config, moe_dispatch, workspace_size
    cfg = S.mini(S.BY_NAME["deepseek_v3_fp8"], T=300, d=512, f=256, E=32).replace(k=4)
    x = S.x(cfg)
    L, idx, _ = oracle.route(cfg, x, S.w_router(cfg))
    counts, offsets, rmap, ptok = oracle.dispatch_index(idx, cfg.E)
    xq, xs = oracle.quant_blocks(oracle.as_f32(x), 1, 128)
    c = make_config(**cfg.describe())
    A = cfg.A
    out = dict(counts=torch.empty(cfg.E, dtype=torch.int32, device=DEV),
               offsets=torch.empty(cfg.E + 1, dtype=torch.int32, device=DEV),
               rmap=torch.empty(cfg.T, cfg.k, dtype=torch.int32, device=DEV),
               ptok=torch.empty(A, dtype=torch.int32, device=DEV),
               xq=torch.empty(A, cfg.d, dtype=torch.uint8, device=DEV),
               xs=torch.empty(A, cfg.d // 128, dtype=torch.float32, device=DEV))
    ws = torch.empty(workspace_size(c, 1), dtype=torch.uint8, device=DEV)
    moe_dispatch(c, x.to(DEV), torch.from_numpy(idx).to(DEV), out["counts"], out["offsets"],
                 out["rmap"], out["ptok"], out["xq"], out["xs"], ws)
    torch.cuda.synchronize()
    assert np.array_equal(_np(out["offsets"]), offsets)
    assert np.array_equal(_np(out["rmap"]), rmap)
    assert np.array_equal(_np(out["xq"]), oracle.permute(xq, rmap))
    assert np.array_equal(_np(out["xs"]), oracle.permute(xs, rmap))


def _route_sigmoid_gates(x, bias=None):
    """moe_route with 16 experts, top-16, sigmoid scores, no renormalisation
    and gate scale 1, so that every gate is the sigmoid of one logit: x
    [T, 128] f32 on the device, w_router the identity on the first 16 hidden
    columns. Returns (logits, idx, gates) on the device."""
    from mixture_experts_layer_gather_amd import make_config, moe_route
    T = x.shape[0]
    c = make_config(T=T, d=128, E=16, k=16, f=128, score="sigmoid", renorm=False, gate_scale=1.0,
                    act="f32", weight="f32")
    wr = torch.zeros(16, 128, dtype=torch.float32, device=DEV)
    wr[:, :16] = torch.eye(16, device=DEV)
    logits = torch.empty(T, 16, dtype=torch.float32, device=DEV)
    idx = torch.empty(T, 16, dtype=torch.int32, device=DEV)
    gate = torch.empty(T, 16, dtype=torch.float32, device=DEV)
    moe_route(c, x, wr, bias, logits, idx, gate)
    return logits, idx, gate


def test_sigmoid_spec_every_fp32_input():
    """The GPU's sigmoid score (1 / (1 + exp_spec(-L)) with an IEEE divide),
    which decides the group choice of DeepSeek-style routing, against the
    oracle's sigmoid_spec bit for bit over every fp32 bit pattern. Finite
    values go in as logits through the identity router (the fp32 FMA
    recurrence then returns each value itself; -0 becomes +0, whose sigmoid
    is the same); infinities and NaNs, for which the recurrence's x * 0
    terms would not vanish, go in as the expert bias of an all-zero token."""
    T = 1 << 22                        # tokens per launch, 16 values each
    per = 16 * T
    zero_tail = torch.zeros(T, 112, dtype=torch.float32, device=DEV)
    nfin = 0
    for lo in range(0, 1 << 32, per):
        bits = np.arange(lo, lo + per, dtype=np.uint64).astype(np.uint32)
        v = bits.view(np.float32).reshape(T, 16)
        finite = np.isfinite(v)
        if not finite.all():
            v = np.where(finite, v, np.float32(0.0))
        want = oracle.sigmoid_spec(v)
        x = torch.cat([torch.from_numpy(v).to(DEV), zero_tail], dim=1)
        _, idx, gate = _route_sigmoid_gates(x)
        w = torch.from_numpy(want.view(np.int32)).to(DEV)
        ok = torch.equal(torch.gather(w, 1, idx.long()), gate.view(torch.int32))
        if not ok:
            got = gate.view(torch.int32).cpu().numpy()
            exp_ = np.take_along_axis(want.view(np.int32), idx.long().cpu().numpy(), axis=1)
            t, j = np.argwhere(got != exp_)[0]
            e = int(idx[t, j])
            raise AssertionError(f"sigmoid of {v[t, e]!r} (bits {int(v[t, e:e+1].view(np.uint32)[0]):#x}): "
                                 f"GPU {got[t, j]:#x}, oracle {exp_[t, j]:#x}")
        nfin += int(finite.sum())
        if lo % (1 << 30) == 0:
            _say(f"[sigmoid] {lo:#x}: ok")
    assert nfin == (1 << 32) - (1 << 24)          # every finite fp32
    # the 2^24 non-finite patterns: +-inf and a spread of NaN payloads
    specials = np.array([0x7F800000, 0xFF800000, 0x7FC00000, 0xFFC00000, 0x7F800001, 0xFF800001,
                         0x7FFFFFFF, 0xFFFFFFFF, 0x7FA00000, 0xFFA00000, 0x7FBFFFFF, 0xFFBFFFFF,
                         0x7FE00000, 0xFFE00000, 0x7F812345, 0xFF812345], dtype=np.uint32)
    b = specials.view(np.float32)
    _, idx, gate = _route_sigmoid_gates(torch.zeros(1, 128, dtype=torch.float32, device=DEV),
                                        bias=torch.from_numpy(b.copy()).to(DEV))
    want = oracle.sigmoid_spec(b)
    got = gate.cpu().numpy()[0]
    for j, e in enumerate(idx.cpu().numpy()[0]):
        if np.isnan(want[e]):
            assert np.isnan(got[j]), hex(specials[e])
        else:
            assert got[j].view(np.int32) == want[e].view(np.int32), hex(specials[e])


# (T, E): 64 experts per workgroup (>= 512 workgroups) and 32 per workgroup,
# with ragged token and expert tiles
ROUTE_TILE_CASES = [(16384, 128), (300, 64), (1000, 96), (8192, 72)]


@pytest.mark.parametrize("T,E", ROUTE_TILE_CASES)
def test_route_logits_tilings(T, E):
    from mixture_experts_layer_gather_amd import make_config, moe_route, workspace_size
    cfg = S.mini(S.BY_NAME["qwen3_skew_bf16"], T=T, d=256, f=128, E=E).replace(k=4)
    _say(f"[route tiles] T={T} E={E}")
    x, wr = S.x(cfg), S.w_router(cfg)
    bias = S.router_bias(cfg)
    L = oracle.router_logits(x, wr, None if bias is None else bias)
    c = make_config(**cfg.describe())
    logits = torch.empty(T, E, dtype=torch.float32, device=DEV)
    idx = torch.empty(T, cfg.k, dtype=torch.int32, device=DEV)
    gate = torch.empty(T, cfg.k, dtype=torch.float32, device=DEV)
    ws = torch.empty(max(1, workspace_size(c, 0)), dtype=torch.uint8, device=DEV)
    moe_route(c, x.to(DEV), wr.to(DEV), None if bias is None else bias.to(DEV), logits, idx, gate, ws=ws)
    torch.cuda.synchronize()
    assert np.array_equal(_np(logits), L)
    assert np.array_equal(_np(idx), oracle.route_select(L, cfg.k))


def _random_routing(T, E, k, seed, skew):
    """k distinct experts per token; skew > 0 draws experts with Zipf-like
    weights (hot experts, some empty ones)."""
    rng = np.random.default_rng(seed)
    w = 1.0 / np.arange(1, E + 1) ** skew
    keys = np.log(rng.random((T, E))) / w  # Efraimidis-Spirakis: top-k = weighted draw without replacement
    return np.argsort(-keys, axis=1, kind="stable")[:, :k].astype(np.int32)


# (T, E, k, skew): ragged last chunks, E up to the 1024 limit, k = E, hot and
# empty experts; up to 32 chunks of 256 tokens the positions kernel derives
# its bases itself, beyond that a separate scan runs
DISPATCH_INDEX_CASES = [(3000, 24, 3, 0.0), (1024, 1024, 8, 1.1), (4096, 8, 8, 0.0),
                        (12000, 16, 4, 1.2), (2000, 600, 2, 0.0), (257, 5, 5, 0.0),
                        (8192, 6, 2, 0.3), (8193, 16, 2, 0.5), (70000, 16, 2, 0.5)]


@pytest.mark.parametrize("T,E,k,skew", DISPATCH_INDEX_CASES)
def test_dispatch_index_paths(T, E, k, skew):
    from mixture_experts_layer_gather_amd import make_config, moe_dispatch, workspace_size
    d = 128
    _say(f"[dispatch index] T={T} E={E} k={k} skew={skew}")
    idx = _random_routing(T, E, k, seed=T * 7 + E, skew=skew)
    counts, offsets, rmap, ptok = oracle.dispatch_index(idx, E)
    x = torch.arange(T * d, dtype=torch.float32).reshape(T, d).to(torch.bfloat16)
    c = make_config(T=T, d=d, E=E, k=k, f=128)
    A = T * k
    out = dict(counts=torch.empty(E, dtype=torch.int32, device=DEV),
               offsets=torch.empty(E + 1, dtype=torch.int32, device=DEV),
               rmap=torch.empty(T, k, dtype=torch.int32, device=DEV),
               ptok=torch.empty(A, dtype=torch.int32, device=DEV),
               xp=torch.empty(A, d, dtype=torch.bfloat16, device=DEV))
    ws = torch.empty(workspace_size(c, 1), dtype=torch.uint8, device=DEV)
    moe_dispatch(c, x.to(DEV), torch.from_numpy(idx).to(DEV), out["counts"], out["offsets"],
                 out["rmap"], out["ptok"], out["xp"], None, ws)
    torch.cuda.synchronize()
    assert np.array_equal(_np(out["counts"]), counts)
    assert np.array_equal(_np(out["offsets"]), offsets)
    assert np.array_equal(_np(out["rmap"]), rmap)
    assert np.array_equal(_np(out["ptok"]), ptok)
    got = out["xp"].view(torch.int16).cpu().numpy()
    assert np.array_equal(got, oracle.permute(x.view(torch.int16).numpy(), rmap))


# (name, base layer, T, d, E, k): the fused route and dispatch, its histogram
# counted by the selection (E >= 128: up to the 1024-expert, top-16 limit)
# and by the dispatch's own pass (fewer experts); both logits kernel
# families (E <= 32, and 32 / 64 experts per workgroup), up to 32 chunks of
# 256 tokens (bases derived in the positions kernel) and beyond (separate
# scan), ragged last chunks, group-limited sigmoid routing, and the FP8 and
# MXFP8 gathers
ROUTE_DISPATCH_CASES = [("qwen3_skew_bf16", 3000, 256, 8, 2), ("qwen3_skew_bf16", 8192, 256, 72, 4),
                        ("qwen3_skew_bf16", 16384, 256, 128, 8), ("qwen3_skew_bf16", 2000, 128, 1024, 16),
                        ("deepseek_v3_bf16", 1000, 256, 256, 8), ("deepseek_v3_bf16", 9000, 256, 128, 8),
                        ("deepseek_v3_fp8", 300, 512, 256, 4), ("deepseek_v3_mxfp8", 777, 256, 128, 8),
                        ("deepseek_v3_mxfp8", 500, 256, 64, 8), ("tiny_fp32", 257, 128, 5, 5),
                        ("deepseek_v3_fp8", 8192, 7168, 256, 8)]  # the full FP8 DeepSeek-style layer


@pytest.mark.parametrize("name,T,d,E,k", ROUTE_DISPATCH_CASES)
def test_route_dispatch_fused(name, T, d, E, k):
    """moe_route_dispatch (the dispatch histogram counted by the top-k
    selection) against the oracle's router and dispatch, every output bit
    for bit (gates to 1e-6); run twice on one workspace, so the second call
    must clear the counts the first left there."""
    from mixture_experts_layer_gather_amd import make_config, moe_route_dispatch, workspace_size
    cfg = S.mini(S.BY_NAME[name], T=T, d=d, f=128, E=E).replace(k=k)
    _say(f"[route+dispatch] {name} T={T} d={d} E={E} k={k}")
    x, wr = S.x(cfg), S.w_router(cfg)
    bias = S.router_bias(cfg)
    L, idx, gates = oracle.route(cfg, x, wr, bias)
    counts, offsets, rmap, ptok = oracle.dispatch_index(idx, E)
    c = make_config(**cfg.describe())
    A = T * k
    fp8, mx = cfg.weight == "fp8", cfg.weight == "mxfp8"
    xs32 = oracle.as_f32(x)
    if fp8:
        xq, xsc = oracle.quant_blocks(xs32, 1, 128)
    elif mx:
        xq, xsc = oracle.quant_mx_rows(xs32)
    out = dict(logits=torch.empty(T, E, dtype=torch.float32, device=DEV),
               idx=torch.empty(T, k, dtype=torch.int32, device=DEV),
               gate=torch.empty(T, k, dtype=torch.float32, device=DEV),
               rmapu8=torch.empty(T, E, dtype=torch.uint8, device=DEV),
               counts=torch.empty(E, dtype=torch.int32, device=DEV),
               offsets=torch.empty(E + 1, dtype=torch.int32, device=DEV),
               rmap=torch.empty(T, k, dtype=torch.int32, device=DEV),
               ptok=torch.empty(A, dtype=torch.int32, device=DEV))
    if fp8 or mx:
        out["xp"] = torch.empty(A, d, dtype=torch.uint8, device=DEV)
        out["xs"] = (torch.empty(A, d // 128, dtype=torch.float32, device=DEV) if fp8
                     else torch.empty(A, d // 32, dtype=torch.uint8, device=DEV))
    else:
        out["xp"] = torch.empty(A, d, dtype=x.dtype, device=DEV)
        out["xs"] = None
    ws = torch.empty(workspace_size(c, 1), dtype=torch.uint8, device=DEV)
    xd, wd = x.to(DEV), wr.to(DEV)
    bd = None if bias is None else bias.to(DEV)
    for rep in range(2):
        moe_route_dispatch(c, xd, wd, bd, out["logits"], out["idx"], out["gate"], out["rmapu8"],
                           out["counts"], out["offsets"], out["rmap"], out["ptok"], out["xp"], out["xs"], ws)
        torch.cuda.synchronize()
        assert np.array_equal(_np(out["logits"]), L), rep
        assert np.array_equal(_np(out["idx"]), idx), rep
        assert oracle.rel_l2(_np(out["gate"]), gates) <= 1e-6, rep
        want_map = np.zeros((T, E), dtype=np.uint8)
        np.put_along_axis(want_map, idx.astype(np.int64), 1, axis=1)
        assert np.array_equal(_np(out["rmapu8"]), want_map), rep
        assert np.array_equal(_np(out["counts"]), counts), rep
        assert np.array_equal(_np(out["offsets"]), offsets), rep
        assert np.array_equal(_np(out["rmap"]), rmap), rep
        assert np.array_equal(_np(out["ptok"]), ptok), rep
        if fp8 or mx:
            assert np.array_equal(_np(out["xp"]), oracle.permute(xq, rmap)), rep
            assert np.array_equal(_np(out["xs"]), oracle.permute(xsc, rmap)), rep
        else:
            isz = torch.int16 if x.dtype == torch.bfloat16 else torch.int32
            got = out["xp"].view(isz).cpu().numpy()
            assert np.array_equal(got, oracle.permute(x.view(isz).numpy(), rmap)), rep


def test_route_dispatch_graph_replay():
    """moe_route_dispatch captured into a HIP graph (the histogram is cleared
    by a kernel, so the graph holds no memset): every replay, after its
    outputs were scribbled over, equals the eager call bit for bit, also
    after an input that routes differently is copied into the captured
    buffer."""
    from mixture_experts_layer_gather_amd import make_config, moe_route_dispatch, workspace_size
    cfg = S.mini(S.BY_NAME["deepseek_v3_fp8"], T=1500, d=256, f=128, E=128).replace(k=8)
    _say("[route+dispatch graph] deepseek_v3_fp8 T=1500 d=256 E=128 k=8")
    c = make_config(**cfg.describe())
    T, d, E, k, A = cfg.T, cfg.d, cfg.E, cfg.k, cfg.T * cfg.k
    wr = S.w_router(cfg).to(DEV)
    bias = S.router_bias(cfg)
    bias = None if bias is None else bias.to(DEV)
    x = S.x(cfg).to(DEV)
    x2 = S.x(cfg.replace(seed_base=cfg.seed_base + 101)).to(DEV)
    names = ("logits", "idx", "gate", "counts", "offsets", "rmap", "ptok", "xp", "xs")
    out = dict(logits=torch.empty(T, E, dtype=torch.float32, device=DEV),
               idx=torch.empty(T, k, dtype=torch.int32, device=DEV),
               gate=torch.empty(T, k, dtype=torch.float32, device=DEV),
               counts=torch.empty(E, dtype=torch.int32, device=DEV),
               offsets=torch.empty(E + 1, dtype=torch.int32, device=DEV),
               rmap=torch.empty(T, k, dtype=torch.int32, device=DEV),
               ptok=torch.empty(A, dtype=torch.int32, device=DEV),
               xp=torch.empty(A, d, dtype=torch.uint8, device=DEV),
               xs=torch.empty(A, d // 128, dtype=torch.float32, device=DEV))
    ws = torch.empty(workspace_size(c, 1), dtype=torch.uint8, device=DEV)
    xin = x.clone()  # the captured input buffer

    def call():
        moe_route_dispatch(c, xin, wr, bias, out["logits"], out["idx"], out["gate"], None, out["counts"],
                           out["offsets"], out["rmap"], out["ptok"], out["xp"], out["xs"], ws)

    def snapshot():
        torch.cuda.synchronize()
        return {n: out[n].clone() for n in names}

    def scribble():
        for n in names:
            out[n].view(torch.uint8).fill_(0xAB)
        ws.fill_(0x5A)

    call()
    eager1 = snapshot()
    xin.copy_(x2)
    call()
    eager2 = snapshot()
    assert not torch.equal(eager1["counts"], eager2["counts"]), "the second input should route differently"
    xin.copy_(x)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for want, tag in ((eager1, "first input"), (eager2, "second input")):
        if tag == "second input":
            xin.copy_(x2)
        for rep in range(3):
            scribble()
            torch.cuda.synchronize()
            g.replay()
            got = snapshot()
            for n in names:
                assert torch.equal(got[n].view(torch.uint8), want[n].view(torch.uint8)), f"{tag} replay {rep}: {n}"


# ------------------------------------------------------------ full sizes

class _L2:
    """Running ||a - b||^2 and ||b||^2 of one tensor, compared piece by piece."""

    def __init__(self):
        self.num = 0.0
        self.den = 0.0

    def add(self, got, want):
        a = np.asarray(got, dtype=np.float64)
        b = np.asarray(want, dtype=np.float64)
        self.num += float(np.sum((a - b) ** 2))
        self.den += float(np.sum(b * b))

    def rel(self):
        return 0.0 if self.den == 0.0 and self.num == 0.0 else float(np.sqrt(self.num / self.den))


OUTPUTS = ("y", "dx", "dw1", "dw2", "dw_router", "d_gate", "out_perm", "dx_perm", "x_perm")


def _full_size_check(cfg):
    """Every element of every output of a full-size layer against the
    oracle, which runs expert by expert (layer_stream) so that it never holds
    a whole weight gradient; and a second GPU step, bitwise equal."""
    _say(f"[full] {cfg.name}: generating inputs")
    inp = _inputs(cfg, threads=16)
    _say(f"[full] {cfg.name}: GPU layer, two steps")
    layer = _gpu_layer(cfg, inp)
    first = {n: getattr(layer, n).clone() for n in OUTPUTS}
    if cfg.shared:
        first.update(s_dw1=layer.s_dw1.clone(), s_dw2=layer.s_dw2.clone())
    cu = lambda t: t.to(DEV)
    layer.step(cu(inp["x"]), cu(inp["dy"]))
    torch.cuda.synchronize()
    for n, v in first.items():
        assert torch.equal(v, getattr(layer, n)), f"{n} differs between two runs"
    del first
    tol = _tol(cfg)
    errs = {n: _L2() for n in ("out_perm", "dx_perm", "dw1", "dw2")}
    empty = []

    def on_expert(e, r0, r1, t):
        if t is None:
            empty.append(e)
            assert not layer.dw1[e].any() and not layer.dw2[e].any(), f"expert {e}: no rows, dW not 0"
            return
        errs["dw1"].add(_np(layer.dw1[e]), t["dw1"])
        errs["dw2"].add(_np(layer.dw2[e]), t["dw2"])
        errs["out_perm"].add(_np(layer.out_perm[r0:r1]), t["out_perm"])
        errs["dx_perm"].add(_np(layer.dx_perm[r0:r1]), t["dx_perm"])
        if e % 32 == 31:
            _say(f"[full] {cfg.name}: oracle, {e + 1} experts; dW1 {errs['dw1'].rel():.2e} "
                 f"dW2 {errs['dw2'].rel():.2e}")

    _say(f"[full] {cfg.name}: oracle, expert by expert")
    ref = oracle.layer_stream(cfg, inp, on_expert=on_expert)
    _check_routing_and_dispatch(cfg, layer, ref)
    ptok = ref["perm_token"]
    if cfg.weight in ("fp8", "mxfp8"):
        assert np.array_equal(_np(layer.x_perm), ref["xq"][ptok]), "fp8 x_perm codes"
        assert np.array_equal(_np(layer.x_scale), ref["x_scale"][ptok]), "fp8 x_perm scales"
    else:
        assert torch.equal(layer.x_perm, cu(inp["x"])[layer.perm_token.long()]), "x_perm"
    pairs = [(n, errs[n].rel()) for n in errs]
    for n in ("y", "d_gate", "dx", "dw_router"):
        pairs.append((n, oracle.rel_l2(_np(getattr(layer, n)), ref[n])))
    if cfg.shared:
        pairs += [("shared_dw1", oracle.rel_l2(_np(layer.s_dw1[0]), ref["shared_dw1"])),
                  ("shared_dw2", oracle.rel_l2(_np(layer.s_dw2[0]), ref["shared_dw2"]))]
    _say(f"[full] {cfg.name}: " + ", ".join(f"{n} {v:.2e}" for n, v in pairs)
         + f"; {len(empty)} empty experts")
    for n, v in pairs:
        assert v <= tol, f"{n}: rel L2 {v:.3e} > {tol}"


@pytest.mark.parametrize("which", ["mixtral_bf16", "deepseek_v3_bf16", "qwen3_skew_bf16", "deepseek_v3_fp8",
                                   "deepseek_v3_mxfp8"])
def test_full_size_layer(which):
    _full_size_check(S.BY_NAME[which])


# ------------------------------------------------ load-balancing aux loss

AUX_CASES = [
    # (T, d, E, k, act, score): ragged last chunk, several experts per lane,
    # chunks of more than 64 tokens (T > 16384), E = 1000 (one split per expert)
    (777, 128, 64, 4, "f32", "softmax"),
    (513, 256, 300, 8, "bf16", "sigmoid"),
    (70000, 128, 16, 2, "f32", "softmax"),
    (300, 128, 1000, 16, "f32", "softmax"),
    (1, 128, 8, 2, "f32", "softmax"),
]


@pytest.mark.parametrize("T,d,E,k,act,score", AUX_CASES)
def test_aux_loss_and_gradient(T, d, E, k, act, score):
    """The auxiliary loss alone: moe_route_aux_loss against the oracle, then
    moe_route_bwd with d_gate = 0, so that dL is only the auxiliary term
    times d_aux, seen through dw_router = dL^T x and dx = dL w_router."""
    from mixture_experts_layer_gather_amd import _lib as L
    coeff, d_aux = 0.01, 2.5
    cfg = S.LayerConfig("aux", 90 + E % 7, T=T, d=d, E=E, k=k, f=128, act=act, weight=act,
                        score=score, renorm=True, std=0.05, aux_coeff=coeff)
    _say(f"[aux] T={T} d={d} E={E} k={k} {act} {score}")
    x, wr = S.x(cfg), S.w_router(cfg)
    Lo, idx, _ = oracle.route(cfg, x, wr)
    c = L.make_config(**cfg.describe())
    at = torch.float32 if act == "f32" else torch.bfloat16
    xd, wd = x.to(DEV), wr.to(DEV)
    logits = torch.empty(T, E, dtype=torch.float32, device=DEV)
    tidx = torch.empty(T, k, dtype=torch.int32, device=DEV)
    gate = torch.empty(T, k, dtype=torch.float32, device=DEV)
    L.moe_route(c, xd, wd, None, logits, tidx, gate)
    ws = torch.empty(max(1, L.workspace_size(c, L.OP_AUX_LOSS)), dtype=torch.uint8, device=DEV)
    loss = torch.full((1,), float("nan"), device=DEV)
    L.moe_route_aux_loss(c, logits, tidx, loss, ws)
    torch.cuda.synchronize()
    assert np.array_equal(_np(logits), Lo) and np.array_equal(_np(tidx), idx)
    want = oracle.aux_loss(Lo, idx, E, coeff)
    err = abs(loss.item() - want) / want
    _say(f"[aux] loss {loss.item():.8f} oracle {want:.8f} rel {err:.2e}")
    assert err <= 1e-5
    dx = torch.zeros(T, d, dtype=at, device=DEV)
    dwr = torch.empty(E, d, dtype=torch.float32, device=DEV)
    wsb = torch.empty(L.workspace_size(c, L.OP_ROUTE_BWD), dtype=torch.uint8, device=DEV)
    L.moe_route_bwd(c, xd, wd, logits, tidx, gate, torch.zeros(T, k, device=DEV), dx, dwr, wsb,
                    d_aux=torch.full((1,), d_aux, device=DEV))
    torch.cuda.synchronize()
    dL = oracle.aux_loss_dlogits(Lo, idx, E, coeff, d_aux)
    dWr, dx_r = oracle.route_bwd(dL, x, wr)
    tol = TOL[act]
    e1, e2 = oracle.rel_l2(_np(dwr), dWr), oracle.rel_l2(_np(dx), dx_r)
    _say(f"[aux] dw_router rel L2 {e1:.2e} dx rel L2 {e2:.2e}")
    assert e1 <= tol and e2 <= tol
    # d_aux = NULL leaves the auxiliary term out: d_gate = 0 then gives zeros
    dx.zero_()
    L.moe_route_bwd(c, xd, wd, logits, tidx, gate, torch.zeros(T, k, device=DEV), dx, dwr, wsb)
    torch.cuda.synchronize()
    assert not dwr.any() and not dx.any()
