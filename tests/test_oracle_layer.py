"""Pins of the oracle's layer arithmetic: dispatch indexing by brute force and
invariants, the expert FFN against torch's matmul/silu, the identity-expert
invariant, and every gradient against torch.autograd in fp64 (an independent
formulation) and central finite differences."""
import numpy as np
import pytest
import torch

import moe_synth as S
import oracle


def _inputs(cfg):
    w1, w2 = S.all_expert_weights(cfg, threads=1)
    inp = dict(x=S.x(cfg), wr=S.w_router(cfg), bias=S.router_bias(cfg), w1=w1, w2=w2,
               dy=S.dy(cfg))
    if cfg.shared:
        inp.update(sw1=S.shared_w1(cfg), sw2=S.shared_w2(cfg))
    return inp


# ---------------------------------------------------------------- dispatch

@pytest.mark.parametrize("T,E,k", [(1, 4, 2), (33, 8, 2), (70, 16, 5), (50, 6, 6), (129, 3, 1)])
def test_dispatch_index_bruteforce(T, E, k):
    rng = np.random.default_rng(T * E + k)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    counts, offsets, rmap, ptok = oracle.dispatch_index(idx, E)
    # brute force: the rows in sorted (expert, token) order
    entries = sorted((int(idx[t, j]), t, j) for t in range(T) for j in range(k))
    for r, (e, t, j) in enumerate(entries):
        assert rmap[t, j] == r and ptok[r] == t
    # invariants
    assert counts.sum() == T * k and offsets[E] == T * k and offsets[0] == 0
    assert np.array_equal(np.diff(offsets), counts)
    assert np.array_equal(np.sort(rmap.ravel()), np.arange(T * k))
    assert np.array_equal(np.bincount(ptok, minlength=T), np.full(T, k))
    for e in range(E):
        seg = ptok[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)                     # tokens ascend
        assert np.all((idx[seg] == e).sum(1) == 1)          # each routed to e


def test_permute_then_unpermute_is_identity():
    rng = np.random.default_rng(0)
    T, E, k, d = 45, 7, 3, 10
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    _, _, rmap, ptok = oracle.dispatch_index(idx, E)
    x = rng.standard_normal((T, d)).astype(np.float32)
    xp = oracle.permute(x, rmap)
    assert np.array_equal(xp, x[ptok])
    for j in range(k):
        assert np.array_equal(xp[rmap[:, j]], x)
    # with k = 1 and gate 1, combine is the inverse permutation
    idx1 = idx[:, :1]
    _, _, rmap1, _ = oracle.dispatch_index(idx1, E)
    y = oracle.combine(oracle.permute(x, rmap1), rmap1, np.ones((T, 1)))
    assert np.array_equal(y, x.astype(np.float64))


# --------------------------------------------------------------------- FFN

def test_ffn_matches_torch_dense_swiglu():
    g = torch.Generator().manual_seed(7)
    X = torch.randn(33, 48, generator=g, dtype=torch.float64)
    W1 = torch.randn(2 * 40, 48, generator=g, dtype=torch.float64) * 0.1
    W2 = torch.randn(48, 40, generator=g, dtype=torch.float64) * 0.1
    GU, H, O = oracle.ffn_fwd(X.numpy(), W1.numpy(), W2.numpy())
    ref = torch.nn.functional.silu(X @ W1[:40].T) * (X @ W1[40:].T)
    assert np.allclose(H, ref.numpy(), rtol=1e-13, atol=1e-15)
    assert np.allclose(O, (ref @ W2.T).numpy(), rtol=1e-12, atol=1e-14)


def test_identity_experts_return_gate_sum_times_x():
    for base, shared_add in [(S.BY_NAME["tiny_fp32"], 0.0), (S.mini(S.BY_NAME["deepseek_v3_bf16"], 40, 64, 32, E=32), 1.0),
                             (S.mini(S.BY_NAME["qwen3_skew_bf16"], 40, 64, 32, E=16), 0.0)]:
        inp = _inputs(base)
        out = oracle.layer(base, inp, identity=True)
        x = oracle.as_f64(inp["x"])
        gsum = out["gates"].sum(1, keepdims=True)
        assert np.allclose(out["y"], (gsum + shared_add) * x, rtol=1e-13, atol=1e-13)
        if base.renorm:
            assert np.allclose(gsum, base.gate_scale, atol=1e-13)


# --------------------------------------------------------------- gradients

def _torch_layer(cfg, inp, idx, L32):
    """Independent fp64 torch formulation of the layer with the oracle's
    selection held fixed; returns leaves and the scalar loss <y, dy>.
    The gates read the fp32 router logits (their value is L32, their
    gradient flows as for x W_r^T + b)."""
    f = cfg.f
    x = torch.tensor(oracle.as_f64(inp["x"]), requires_grad=True)
    wr = torch.tensor(oracle.as_f64(inp["wr"]), requires_grad=True)
    w1 = torch.tensor(oracle.as_f64(inp["w1"]), requires_grad=True)
    w2 = torch.tensor(oracle.as_f64(inp["w2"]), requires_grad=True)
    L = x @ wr.T
    if inp.get("bias") is not None:
        L = L + torch.tensor(oracle.as_f64(inp["bias"]))
    L = L + (torch.tensor(L32, dtype=torch.float64) - L.detach())
    I = torch.tensor(idx, dtype=torch.int64)
    sel = torch.gather(L, 1, I)
    if cfg.score == "softmax":
        g = torch.softmax(sel, 1) if cfg.renorm else torch.gather(torch.softmax(L, 1), 1, I)
    else:
        s = torch.sigmoid(sel)
        g = s / s.sum(1, keepdim=True) if cfg.renorm else s
    g = g * cfg.gate_scale
    y = torch.zeros_like(x)
    for t in range(x.shape[0]):
        for j in range(cfg.k):
            e = int(idx[t, j])
            gu = w1[e] @ x[t]
            h = torch.nn.functional.silu(gu[:f]) * gu[f:]
            y[t] = y[t] + g[t, j] * (w2[e] @ h)
    leaves = dict(x=x, wr=wr, w1=w1, w2=w2)
    if cfg.shared:
        sw1 = torch.tensor(oracle.as_f64(inp["sw1"]), requires_grad=True)
        sw2 = torch.tensor(oracle.as_f64(inp["sw2"]), requires_grad=True)
        gu = x @ sw1.T
        y = y + (torch.nn.functional.silu(gu[:, :f]) * gu[:, f:]) @ sw2.T
        leaves.update(sw1=sw1, sw2=sw2)
    loss = (y * torch.tensor(oracle.as_f64(inp["dy"]))).sum()
    return leaves, y, loss


@pytest.mark.parametrize("which", ["tiny_fp32", "deepseek_v3_bf16", "qwen3_skew_bf16"])
def test_layer_matches_torch_autograd_fp64(which):
    cfg = S.BY_NAME[which]
    if which != "tiny_fp32":
        cfg = S.mini(cfg, T=24, d=32, f=24, E=16 if which == "deepseek_v3_bf16" else 8)
        if which == "deepseek_v3_bf16":
            cfg = cfg.replace(num_groups=4, topk_groups=2, k=3)
        else:
            cfg = cfg.replace(k=3)
    else:
        cfg = S.mini(cfg, T=30, d=24, f=20)
    inp = _inputs(cfg)
    out = oracle.layer(cfg, inp)
    leaves, y, loss = _torch_layer(cfg, inp, out["idx"], out["logits"])
    loss.backward()
    assert np.allclose(out["y"], y.detach().numpy(), rtol=1e-12, atol=1e-14)
    assert np.allclose(out["dx"], leaves["x"].grad.numpy(), rtol=1e-10, atol=1e-13)
    assert np.allclose(out["dw_router"], leaves["wr"].grad.numpy(), rtol=1e-10, atol=1e-13)
    assert np.allclose(out["dw1"], leaves["w1"].grad.numpy(), rtol=1e-10, atol=1e-13)
    assert np.allclose(out["dw2"], leaves["w2"].grad.numpy(), rtol=1e-10, atol=1e-13)
    if cfg.shared:
        assert np.allclose(out["shared_dw1"], leaves["sw1"].grad.numpy(), rtol=1e-10, atol=1e-13)
        assert np.allclose(out["shared_dw2"], leaves["sw2"].grad.numpy(), rtol=1e-10, atol=1e-13)


def test_layer_gradients_central_differences():
    """Central differences of <y, dy> in fp64 with routing frozen; the
    selection margin is checked to exceed the perturbation's effect."""
    cfg = S.mini(S.BY_NAME["tiny_fp32"], T=12, d=16, f=12, E=4)
    inp = _inputs(cfg)
    out = oracle.layer(cfg, inp)
    L = out["logits"].astype(np.float64)
    srt = np.sort(L, axis=1)
    margin = np.min(srt[:, -cfg.k] - srt[:, -cfg.k - 1])
    assert margin > 1e-6
    dy = oracle.as_f64(inp["dy"])
    idx = out["idx"]

    def loss(x, wr, w1, w2):
        Lx = x @ wr.T
        g = oracle.route_gates(Lx, idx, cfg.score, cfg.renorm, cfg.gate_scale)
        _, _, rmap, _ = oracle.dispatch_index(idx, cfg.E)
        Xp = oracle.permute(x, rmap)
        _, offs, _, _ = oracle.dispatch_index(idx, cfg.E)
        O = np.zeros((cfg.A, cfg.d))
        for e in range(cfg.E):
            r0, r1 = offs[e], offs[e + 1]
            if r1 > r0:
                O[r0:r1] = oracle.ffn_fwd(Xp[r0:r1], w1[e], w2[e])[2]
        return float((oracle.combine(O, rmap, g) * dy).sum())

    base = dict(x=oracle.as_f64(inp["x"]), wr=oracle.as_f64(inp["wr"]),
                w1=oracle.as_f64(inp["w1"]), w2=oracle.as_f64(inp["w2"]))
    grads = dict(x=out["dx"], wr=out["dw_router"], w1=out["dw1"], w2=out["dw2"])
    rng = np.random.default_rng(0)
    h = 1e-6
    for name in base:
        for _ in range(6):
            pos = tuple(int(rng.integers(0, s)) for s in base[name].shape)
            p = {kk: v.copy() for kk, v in base.items()}
            p[name][pos] += h
            lp = loss(**p)
            p[name][pos] -= 2 * h
            lm = loss(**p)
            fd = (lp - lm) / (2 * h)
            assert abs(fd - grads[name][pos]) <= 1e-6 * max(1.0, abs(fd)), (name, pos, fd, grads[name][pos])


def test_fp8_layer_consistency():
    """fp8 weights: the oracle's own quantisation of the bf16 masters is used
    consistently and stays close to the unquantised layer."""
    cfg = S.mini(S.BY_NAME["deepseek_v3_fp8"], T=16, d=256, f=256, E=16).replace(num_groups=4, topk_groups=2, k=4)
    inp = _inputs(cfg)
    out = oracle.layer(cfg, inp)
    ref = oracle.layer(cfg.replace(weight="bf16"), inp)
    assert np.array_equal(out["idx"], ref["idx"])
    assert oracle.rel_l2(out["y"], ref["y"]) < 0.08
    q1, s1, q2, s2 = out["w_q"][3]
    assert s1.shape == (2 * cfg.f // 128, cfg.d // 128) and s2.shape == (cfg.d // 128, cfg.f // 128)


# ------------------------------------------ load-balancing auxiliary loss

def test_aux_loss_balanced_routing_equals_coefficient():
    # equal logits (p = 1/E) and every expert holding T k / E slots (f = 1/E):
    # coeff * E * sum_e (1/E)(1/E) = coeff exactly
    E, T, k = 8, 16, 2
    L = np.zeros((T, E), dtype=np.float32)
    idx = np.array([[(2 * t) % E, (2 * t + 1) % E] for t in range(T)], dtype=np.int32)
    assert oracle.aux_loss(L, idx, E, 0.01) == pytest.approx(0.01, rel=1e-15)


def test_aux_loss_two_experts_closed_form():
    # one token, two experts, slot on expert 0: loss = 2 c sigma(a - b),
    # dloss/da = -dloss/db = 2 c p0 p1
    a, b, c = 0.7, -0.4, 0.03
    L = np.array([[a, b]], dtype=np.float64)
    idx = np.array([[0]], dtype=np.int32)
    p0 = 1.0 / (1.0 + np.exp(-(a - b)))
    assert oracle.aux_loss(L, idx, 2, c) == pytest.approx(2 * c * p0, rel=1e-14)
    g = oracle.aux_loss_dlogits(L, idx, 2, c)
    assert g[0, 0] == pytest.approx(2 * c * p0 * (1 - p0), rel=1e-12)
    assert g[0, 1] == pytest.approx(-2 * c * p0 * (1 - p0), rel=1e-12)


def test_aux_loss_gradient_matches_autograd_and_differences():
    rng = np.random.default_rng(5)
    T, E, k, c, d_aux = 40, 12, 3, 0.01, 1.7
    L = rng.normal(size=(T, E)) * 2.0
    idx = np.argsort(-L, axis=1)[:, :k].astype(np.int32)
    g = oracle.aux_loss_dlogits(L, idx, E, c, d_aux)
    # torch autograd on an independent formulation (f constant)
    f = torch.bincount(torch.from_numpy(idx.astype(np.int64)).reshape(-1), minlength=E).double() / (T * k)
    Lt = torch.from_numpy(L).requires_grad_(True)
    loss = c * E * (f * torch.softmax(Lt, dim=1).mean(dim=0)).sum()
    (d_aux * loss).backward()
    assert np.allclose(g, Lt.grad.numpy(), rtol=1e-12, atol=1e-15)
    assert oracle.aux_loss(L, idx, E, c) == pytest.approx(float(loss), rel=1e-13)
    # central differences of the oracle's own loss (selection held fixed)
    h = 1e-6
    for t, e in [(0, 0), (7, 5), (39, 11)]:
        Lp, Lm = L.copy(), L.copy()
        Lp[t, e] += h
        Lm[t, e] -= h
        fd = (oracle.aux_loss(Lp, idx, E, c) - oracle.aux_loss(Lm, idx, E, c)) / (2 * h)
        assert d_aux * fd == pytest.approx(g[t, e], rel=1e-5, abs=1e-11)
    # softmax is shift invariant: every row of the gradient sums to zero
    assert np.allclose(g.sum(axis=1), 0.0, atol=1e-15)


def _mx_mini():
    return S.mini(S.BY_NAME["deepseek_v3_mxfp8"], T=16, d=256, f=256, E=16).replace(
        num_groups=4, topk_groups=2, k=4)


def test_mxfp8_layer_plumbing_reduces_to_unquantised(monkeypatch):
    """With every MX quantise-dequantise replaced by the identity, the mxfp8
    layer must equal the unquantised one up to the fp32 rounding that H, dO
    and [dG dU] take before quantisation (relative 1e-7): each product then
    takes the operands it would take without quantisation (no transposed or
    swapped weights, no gradient quantised where it should not be), which
    any plumbing mistake would break at order 1."""
    cfg = _mx_mini()
    inp = _inputs(cfg)
    ref = oracle.layer(cfg.replace(weight="bf16", quant_block=128), inp)
    ident = lambda a: (np.asarray(a, dtype=np.float32), None)
    monkeypatch.setattr(oracle, "quant_mx_rows", ident)
    monkeypatch.setattr(oracle, "quant_mx_cols", ident)
    monkeypatch.setattr(oracle, "dequant_mx_rows", lambda q, e: q.astype(np.float64))
    monkeypatch.setattr(oracle, "dequant_mx_cols", lambda q, e: q.astype(np.float64))
    monkeypatch.setattr(oracle, "mx_roundtrip_rows", lambda a: np.asarray(a, np.float32).astype(np.float64))
    out = oracle.layer(cfg, inp)
    for n in ("y", "dx", "dw1", "dw2", "dw_router", "d_gate", "shared_dw1", "shared_dw2"):
        assert oracle.rel_l2(out[n], ref[n]) < 1e-6, n


def test_mxfp8_layer_close_to_unquantised():
    cfg = _mx_mini()
    inp = _inputs(cfg)
    out = oracle.layer(cfg, inp)
    ref = oracle.layer(cfg.replace(weight="bf16", quant_block=128), inp)
    assert np.array_equal(out["idx"], ref["idx"])
    for n in ("y", "dx", "dw1", "dw2", "shared_dw1", "shared_dw2"):
        assert oracle.rel_l2(out[n], ref[n]) < 0.1, n
    wq = out["w_q"][3]
    f, d = cfg.f, cfg.d
    assert wq["w1_rows"][1].shape == (2 * f, d // 32) and wq["w2_rows"][1].shape == (d, f // 32)
    assert wq["w1_cols"][1].shape == (2 * f // 32, d) and wq["w2_cols"][1].shape == (d // 32, f)
    assert out["x_scale"].dtype == np.uint8 and out["x_scale"].shape == (cfg.T, d // 32)


def test_mxfp8_column_blocks_feed_only_the_data_gradients(monkeypatch):
    """Marking the column-quantised weights (dequantised x2, exact) must
    double dH and so dW1, quadruple dX through both data-gradient products,
    and leave y and dW2 unchanged: the 32 x 1 weight blocks serve exactly
    the two data-gradient products."""
    cfg = _mx_mini()
    inp = _inputs(cfg)
    ident = lambda a: (np.asarray(a, dtype=np.float32), None)
    monkeypatch.setattr(oracle, "quant_mx_rows", ident)
    monkeypatch.setattr(oracle, "quant_mx_cols", ident)
    monkeypatch.setattr(oracle, "dequant_mx_rows", lambda q, e: q.astype(np.float64))
    monkeypatch.setattr(oracle, "mx_roundtrip_rows", lambda a: np.asarray(a, np.float32).astype(np.float64))
    monkeypatch.setattr(oracle, "dequant_mx_cols", lambda q, e: q.astype(np.float64))
    # the weight-gradient token blocks are column blocks too: held fixed here
    monkeypatch.setattr(oracle, "mx_roundtrip_tokens", lambda a: np.asarray(a, np.float32).astype(np.float64))
    base = oracle.layer(cfg, inp)
    monkeypatch.setattr(oracle, "dequant_mx_cols", lambda q, e: 2.0 * q.astype(np.float64))
    out = oracle.layer(cfg, inp)
    assert np.array_equal(out["y"], base["y"]) and np.array_equal(out["dw2"], base["dw2"])
    assert oracle.rel_l2(out["dw1"], 2 * base["dw1"]) < 1e-6
    assert oracle.rel_l2(out["dx_perm"], 4 * base["dx_perm"]) < 1e-6
    assert oracle.rel_l2(out["shared_dx"], 4 * base["shared_dx"]) < 1e-6


# ------------------------- FP8 weight gradients on 128-row x 1 blocks

def test_fp8_token_blocks_are_row_blocks_of_the_transpose():
    """128-row x 1 blocks from the first row (ragged tail kept short) are the
    1 x 128 row blocks of the transpose, and zero-padding the tail to a whole
    block changes no kept value."""
    rng = np.random.default_rng(21)
    a = (rng.normal(size=(300, 40)) * np.exp(rng.normal(size=(1, 40)) * 3)).astype(np.float32)
    a[128:256, 7] = 0.0                                  # an all-zero block
    got = oracle.fp8_roundtrip_tokens(a)
    assert np.array_equal(got, oracle.fp8_roundtrip_rows(np.ascontiguousarray(a.T)).T)
    padded = np.concatenate([a, np.zeros((84, 40), np.float32)])
    assert np.array_equal(oracle.fp8_roundtrip_tokens(padded)[:300], got)
    assert not got[128:256, 7].any()
    # each block's largest magnitude takes the largest code, 448 x its
    # block's scale (amax / 448 in fp32): the block boundaries are the ones
    # the amax came from
    for b0, b1 in ((0, 128), (128, 256), (256, 300)):
        blk = np.abs(a[b0:b1])
        i = blk.argmax(axis=0)
        c = np.arange(40)
        amax = blk[i, c]
        scale = np.where(amax == 0, np.float32(1), amax / np.float32(448)).astype(np.float32)
        want = np.where(amax == 0, 0.0, 448.0 * scale.astype(np.float64))
        assert np.array_equal(np.abs(got[b0:b1][i, c]), want)
    # relative error of an E4M3 rounding: at most 2^-4 of the block's amax
    amax = np.stack([np.abs(a[b0:b1]).max(0) for b0, b1 in ((0, 128), (128, 256), (256, 300))])
    bound = np.repeat(amax, [128, 128, 44], axis=0) * 2.0 ** -4
    assert np.all(np.abs(got - a) <= bound)


def test_fp8_wgrad_token_blocks_feed_only_the_weight_gradients(monkeypatch):
    """With the 128-row quantiser replaced by an exact doubling, the FP8
    layer's dW1 and dW2 (both operands marked) become 4x those of the
    unquantised-gradient reading and nothing else moves: the token blocks
    serve exactly the four operands of the two weight-gradient products."""
    cfg = S.mini(S.BY_NAME["deepseek_v3_fp8"], T=40, d=256, f=256, E=8).replace(num_groups=4, topk_groups=2, k=4)
    inp = _inputs(cfg)
    base = oracle.layer(cfg, inp, fp8_wgrad=False)
    monkeypatch.setattr(oracle, "fp8_roundtrip_tokens", lambda a: 2.0 * np.asarray(a, np.float64))
    out = oracle.layer(cfg, inp, fp8_wgrad=True)
    for n in ("y", "dx", "dx_perm", "d_gate", "dw_router", "shared_dx"):
        assert np.array_equal(out[n], base[n]), n
    for n in ("dw1", "dw2", "shared_dw1", "shared_dw2"):
        assert oracle.rel_l2(out[n], 4.0 * base[n]) < 1e-14, n
    # and with the identity in its place both readings coincide (up to the
    # fp32 rounding the quantiser's input takes)
    monkeypatch.setattr(oracle, "fp8_roundtrip_tokens",
                        lambda a: np.asarray(a, np.float32).astype(np.float64))
    out = oracle.layer(cfg, inp, fp8_wgrad=True)
    for n in ("dw1", "dw2", "shared_dw1", "shared_dw2"):
        assert oracle.rel_l2(out[n], base[n]) < 1e-7, n


def test_fp8_wgrad_token_blocks_close_to_unquantised_gradients():
    cfg = S.mini(S.BY_NAME["deepseek_v3_fp8"], T=300, d=256, f=256, E=4).replace(num_groups=2, topk_groups=1, k=2)
    inp = _inputs(cfg)
    a = oracle.layer(cfg, inp, fp8_wgrad=False)
    b = oracle.layer(cfg, inp, fp8_wgrad=True)
    assert np.array_equal(a["y"], b["y"]) and np.array_equal(a["dx"], b["dx"])
    for n in ("dw1", "dw2", "shared_dw1", "shared_dw2"):
        err = oracle.rel_l2(b[n], a[n])
        assert 1e-3 < err < 0.06, (n, err)


# ------------------------- MXFP8 weight gradients on 32-row x 1 blocks

def _mx_exp_brute(amax):
    """Smallest integer x in [-127, 127] with amax * 2^-x <= 448, by search."""
    if amax == 0:
        return 0
    for x in range(-127, 128):
        if float(amax) * 2.0 ** -x <= 448.0:
            return x
    raise AssertionError


def test_mx_token_blocks_follow_the_expert_rows():
    """32-row x 1 blocks from the first row, ragged tail kept short: they are
    the 1 x 32 row blocks of the zero-padded transpose, padding changes no
    kept value, and each block's largest magnitude picks the block's
    power-of-two scale (brute-force exponent search) and lands in
    [224, 448] x that scale: the block boundaries are the ones the scales
    came from."""
    rng = np.random.default_rng(31)
    M, C = 75, 40
    a = (rng.normal(size=(M, C)) * np.exp(rng.normal(size=(1, C)) * 3)).astype(np.float32)
    a[32:64, 7] = 0.0                                    # an all-zero block
    a[40, 9] = 1e4                                       # one large element
    got = oracle.mx_roundtrip_tokens(a)
    assert got.shape == (M, C)
    pad = np.concatenate([a, np.zeros((96 - M, C), np.float32)])
    assert np.array_equal(got, oracle.mx_roundtrip_rows(np.ascontiguousarray(pad.T)).T[:M])
    assert np.array_equal(oracle.mx_roundtrip_tokens(pad)[:M], got)
    assert not got[32:64, 7].any()
    for b0, b1 in ((0, 32), (32, 64), (64, M)):
        for c in range(C):
            blk = a[b0:b1, c]
            x = _mx_exp_brute(np.max(np.abs(blk)))
            scaled = np.abs(got[b0:b1, c]) * 2.0 ** -x
            assert np.all(scaled <= 448.0)
            if blk.any():
                assert 224.0 <= scaled.max(), (b0, c)
    # the large element sets its own block's scale only
    assert np.abs(got[32:64, 9]).max() >= 224.0 * 2.0 ** _mx_exp_brute(1e4)
    assert np.abs(got[0:32, 9]).max() < 2.0 ** _mx_exp_brute(1e4)


def test_mx_wgrad_token_blocks_feed_only_the_weight_gradients(monkeypatch):
    """With the 32-row quantiser replaced by an exact doubling, the MXFP8
    layer's dW1 and dW2 (both operands marked) become 4x those of the
    unquantised-gradient reading and nothing else moves; with the identity
    in its place both readings coincide."""
    cfg = _mx_mini().replace(T=40)
    inp = _inputs(cfg)
    base = oracle.layer(cfg, inp, fp8_wgrad=False)
    monkeypatch.setattr(oracle, "mx_roundtrip_tokens", lambda a: 2.0 * np.asarray(a, np.float64))
    out = oracle.layer(cfg, inp, fp8_wgrad=True)
    for n in ("y", "dx", "dx_perm", "d_gate", "dw_router", "shared_dx"):
        assert np.array_equal(out[n], base[n]), n
    for n in ("dw1", "dw2", "shared_dw1", "shared_dw2"):
        assert oracle.rel_l2(out[n], 4.0 * base[n]) < 1e-14, n
    monkeypatch.setattr(oracle, "mx_roundtrip_tokens",
                        lambda a: np.asarray(a, np.float32).astype(np.float64))
    out = oracle.layer(cfg, inp, fp8_wgrad=True)
    for n in ("dw1", "dw2", "shared_dw1", "shared_dw2"):
        assert oracle.rel_l2(out[n], base[n]) < 1e-7, n


def test_mx_wgrad_token_blocks_close_to_unquantised_gradients():
    cfg = _mx_mini().replace(T=300, E=4, num_groups=2, topk_groups=1, k=2)
    inp = _inputs(cfg)
    a = oracle.layer(cfg, inp, fp8_wgrad=False)
    b = oracle.layer(cfg, inp, fp8_wgrad=True)
    assert np.array_equal(a["y"], b["y"]) and np.array_equal(a["dx"], b["dx"])
    for n in ("dw1", "dw2", "shared_dw1", "shared_dw2"):
        err = oracle.rel_l2(b[n], a[n])
        assert 1e-3 < err < 0.06, (n, err)
