"""CPU oracle of the MoE layer token path, forward and backward.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package. It shares no
code with the GPU library (``mixture_experts_layer_gather_amd``) and never
imports it.

Everything floating-point is computed in float64 on the values as stored
(bf16/fp32 inputs widened exactly), except the two pieces that must be
reproduced bit for bit and are therefore specified in fp32 and implemented
in plain C (``spec.c``): the router logits and the selection that reads them
(including the sigmoid group score and its exponential ``exp_spec``), the
FP8 E4M3 block quantiser with fp32 scales, and the MXFP8 quantiser (E4M3
codes in blocks of 32 with power-of-two E8M0 scales).

Sources. The pages name the stages and their meaning, not their formulas:
  * router -> a few experts per token, the rest idle
    (Megatron Core MoE summary, "O essencial"; technical summary section 1);
  * dispatch sends tokens to their experts following the routing map and
    combine brings them back with high-precision accumulation
    (Hybrid-EP article, section on the Hybrid-EP design);
  * dropless MoE, device-read dynamic shapes, grouped GEMM, fused routing and
    permutation (Megatron Core MoE summary, section 2.4);
  * memory-efficient permutation: no redundant intermediate tensors
    (Megatron Core MoE summary, section 2.2).
The formulas (softmax or sigmoid scores, top-k, renormalisation, the group
limit, the 2.5 gate scale, SwiGLU experts, the FP8 block sizes) come from
the five workload definitions; every reading the pages leave open is listed
beside the function that takes it.

Parity pins: every function here is checked in ``tests/test_oracle_*.py``
against brute force, closed forms, invariants or library routines.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "spec.c")
_SO = os.path.join(_HERE, "liboracle_spec.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C part of the oracle with gcc (no fused contraction)."""
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math",
                               "-fopenmp", "-fPIC", "-shared", "-std=c11", _SRC,
                               "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        L.orc_exp_spec.restype = ctypes.c_float
        L.orc_exp_spec.argtypes = [ctypes.c_float]
        L.orc_sigmoid_spec.restype = ctypes.c_float
        L.orc_sigmoid_spec.argtypes = [ctypes.c_float]
        L.orc_exp_spec_array.argtypes = [P, P, i64]
        L.orc_sigmoid_spec_array.argtypes = [P, P, i64]
        L.orc_exp_spec_max_ulp.restype = ctypes.c_double
        L.orc_exp_spec_max_ulp.argtypes = [ctypes.c_uint32, ctypes.c_uint32,
                                           ctypes.POINTER(ctypes.c_int64)]
        L.orc_router_logits.argtypes = [i64, i64, i64, P, P, P, P]
        L.orc_route_select.restype = ctypes.c_int
        L.orc_route_select.argtypes = [i64, i64, i64, P, i64, i64, ctypes.c_int, P]
        L.orc_e4m3_encode.restype = ctypes.c_uint8
        L.orc_e4m3_encode.argtypes = [ctypes.c_float]
        L.orc_e4m3_decode.restype = ctypes.c_float
        L.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_encode_array.argtypes = [P, P, i64]
        L.orc_e4m3_decode_array.argtypes = [P, P, i64]
        L.orc_quant_blocks.argtypes = [i64, i64, P, i64, i64, P, P]
        L.orc_mx_scale_exp.restype = ctypes.c_int
        L.orc_mx_scale_exp.argtypes = [ctypes.c_float]
        L.orc_quant_mx_rows.argtypes = [i64, i64, P, P, P]
        L.orc_quant_mx_cols.argtypes = [i64, i64, P, P, P]
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def as_f32(a) -> np.ndarray:
    """Exact widening of stored values (fp32 or bf16 torch/numpy) to fp32."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            return np.ascontiguousarray(a.detach().to("cpu", torch.float32).numpy())
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def as_f64(a) -> np.ndarray:
    """Exact widening of stored values to fp64."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            return np.ascontiguousarray(a.detach().to("cpu", torch.float64).numpy())
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(a, dtype=np.float64)


# ------------------------------------------------------------ fp32 specs

def exp_spec(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty_like(x)
    lib().orc_exp_spec_array(_ptr(x), _ptr(out), x.size)
    return out


def sigmoid_spec(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty_like(x)
    lib().orc_sigmoid_spec_array(_ptr(x), _ptr(out), x.size)
    return out


def router_logits(x, wr, bias=None) -> np.ndarray:
    """L[t,e] = sum_i x[t,i] w[e,i] as an fp32 sequential FMA in ascending i,
    then + bias[e] in fp32. Reading: the pages give no router precision;
    ranking must be reproducible, so the order is fixed."""
    x = as_f32(x)
    wr = as_f32(wr)
    T, d = x.shape
    E = wr.shape[0]
    b = as_f32(bias) if bias is not None else None
    out = np.empty((T, E), dtype=np.float32)
    lib().orc_router_logits(T, d, E, _ptr(x), _ptr(wr), _ptr(b), _ptr(out))
    return out


GROUP_SCORE = {"top2_sum": 0, "max": 1}


def route_select(logits, k: int, num_groups: int = 1, topk_groups: int = 1,
                 group_score: str = "top2_sum") -> np.ndarray:
    """Top-k expert indices per token, slots in rank order (larger logit
    first, ties to the lower expert index), with the optional group limit."""
    L = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = L.shape
    idx = np.empty((T, k), dtype=np.int32)
    rc = lib().orc_route_select(T, E, k, _ptr(L), num_groups, topk_groups,
                                GROUP_SCORE[group_score], _ptr(idx))
    if rc != 0:
        raise ValueError("bad routing arguments")
    return idx


def route_scores(logits, score: str) -> np.ndarray:
    """Per-expert scores in fp64 from the fp32 logits: softmax over all
    experts (max-subtracted) or the logistic sigmoid."""
    L = np.asarray(logits, dtype=np.float64)
    if score == "softmax":
        z = np.exp(L - L.max(axis=1, keepdims=True))
        return z / z.sum(axis=1, keepdims=True)
    if score == "sigmoid":
        return 1.0 / (1.0 + np.exp(-L))
    raise ValueError(score)


def route_gates(logits, idx, score: str, renorm: bool, gate_scale: float) -> np.ndarray:
    """Gate of each selected slot, fp64.
      softmax, renorm: softmax over the selected logits (= p_j / sum_sel p)
      softmax, plain : p_{e_j}, the softmax over all experts
      sigmoid, renorm: s_j / sum_sel s
      sigmoid, plain : s_j
    each times gate_scale."""
    L = np.asarray(logits, dtype=np.float64)
    sel = np.take_along_axis(L, idx.astype(np.int64), axis=1)
    if score == "softmax":
        if renorm:
            z = np.exp(sel - sel.max(axis=1, keepdims=True))
            g = z / z.sum(axis=1, keepdims=True)
        else:
            g = np.take_along_axis(route_scores(L, "softmax"), idx.astype(np.int64), axis=1)
    elif score == "sigmoid":
        s = 1.0 / (1.0 + np.exp(-sel))
        g = s / s.sum(axis=1, keepdims=True) if renorm else s
    else:
        raise ValueError(score)
    return g * gate_scale


def route(cfg, x, wr, bias=None):
    """Router forward for a layer config: (logits fp32, idx int32, gates fp64)."""
    L = router_logits(x, wr, bias)
    idx = route_select(L, cfg.k, cfg.num_groups, cfg.topk_groups, cfg.group_score)
    g = route_gates(L, idx, cfg.score, cfg.renorm, cfg.gate_scale)
    return L, idx, g


# ------------------------------------------------------- dispatch indexing

def dispatch_index(idx, E: int):
    """Expert-contiguous row order: rows sorted by (expert, token), slots of
    one token never share an expert.
      counts[e]      number of (t, j) with idx[t,j] == e
      offsets[e]     exclusive prefix sum of counts, offsets[E] = T*k
      row_id_map[t,j] = offsets[e] + #{t' < t : e in idx[t']}
      perm_token[r]  source token of row r
    A stable sort of the flattened index list gives exactly this order."""
    idx = np.asarray(idx, dtype=np.int64)
    T, k = idx.shape
    flat = idx.reshape(-1)
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    order = np.argsort(flat, kind="stable")      # row r -> flat entry t*k+j
    row_id_map = np.empty(T * k, dtype=np.int32)
    row_id_map[order] = np.arange(T * k, dtype=np.int32)
    perm_token = (order // k).astype(np.int32)
    return counts, offsets, row_id_map.reshape(T, k), perm_token


def permute(x, row_id_map) -> np.ndarray:
    """x_perm[row_id_map[t,j]] = x[t] (exact copy, any dtype)."""
    x = np.asarray(x)
    T, k = row_id_map.shape
    out = np.empty((T * k,) + x.shape[1:], dtype=x.dtype)
    for j in range(k):
        out[row_id_map[:, j]] = x
    return out


# -------------------------------------------------------------- fp8 E4M3

def e4m3_encode(v) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    lib().orc_e4m3_encode_array(_ptr(v), _ptr(out), v.size)
    return out


def e4m3_decode(c) -> np.ndarray:
    c = np.ascontiguousarray(c, dtype=np.uint8)
    out = np.empty(c.shape, dtype=np.float32)
    lib().orc_e4m3_decode_array(_ptr(c), _ptr(out), c.size)
    return out


def quant_blocks(src, br: int, bc: int):
    """Block FP8 quantisation: returns (q uint8 [R,C], scale fp32 [R/br, C/bc])."""
    s = as_f32(src)
    R, C = s.shape
    q = np.empty((R, C), dtype=np.uint8)
    sc = np.empty(((R + br - 1) // br, (C + bc - 1) // bc), dtype=np.float32)
    lib().orc_quant_blocks(R, C, _ptr(s), br, bc, _ptr(q), _ptr(sc))
    return q, sc


def dequant_blocks(q, scale, br: int, bc: int) -> np.ndarray:
    """float(q) * scale, exact in fp64."""
    v = e4m3_decode(q).astype(np.float64)
    R, C = v.shape
    s = np.repeat(np.repeat(np.asarray(scale, np.float64), br, axis=0)[:R], bc, axis=1)[:, :C]
    return v * s


def fp8_roundtrip_rows(a, block: int = 128) -> np.ndarray:
    """Quantise rows in 1 x block blocks (from fp32) and dequantise (fp64)."""
    q, s = quant_blocks(np.asarray(a, dtype=np.float32), 1, block)
    return dequant_blocks(q, s, 1, block)


def fp8_roundtrip_tokens(a, block: int = 128) -> np.ndarray:
    """Quantise one expert's rows [M, C] (from fp32) in blocks of `block`
    consecutive rows x 1 column and dequantise (fp64): the operands of a
    weight-gradient product, whose contraction runs over the expert's rows.
    The blocks start at the expert's first row; the last one holds the
    M mod block remaining rows, which is what zero-padding it to a whole
    block would give (zeros change neither the amax nor the kept codes)."""
    q, s = quant_blocks(np.asarray(a, dtype=np.float32), block, 1)
    return dequant_blocks(q, s, block, 1)


# ------------------------------------------------------------ MXFP8

MX_BLOCK = 32


def quant_mx_rows(src):
    """MXFP8 quantisation of the rows of src [R,C] (C a multiple of 32) in
    1 x 32 blocks: returns (q uint8 [R,C] E4M3 codes, e8m0 uint8 [R,C/32]).
    The rule (OCP MX v1.0) is in spec.c: orc_quant_mx_rows."""
    s = as_f32(src)
    R, C = s.shape
    if C % MX_BLOCK:
        raise ValueError("MXFP8 rows need a multiple of 32 columns")
    q = np.empty((R, C), dtype=np.uint8)
    e = np.empty((R, C // MX_BLOCK), dtype=np.uint8)
    lib().orc_quant_mx_rows(R, C, _ptr(s), _ptr(q), _ptr(e))
    return q, e


def quant_mx_cols(src):
    """MXFP8 in 32 x 1 blocks (32 consecutive rows of one column), for an
    operand contracted over its rows: (q uint8 [R,C], e8m0 uint8 [R/32, C]),
    the row rule applied to the transpose (spec.c: orc_quant_mx_cols walks
    the columns in place)."""
    s = as_f32(src)
    R, C = s.shape
    if R % MX_BLOCK:
        raise ValueError("MXFP8 column blocks need a multiple of 32 rows")
    q = np.empty((R, C), dtype=np.uint8)
    e = np.empty((R // MX_BLOCK, C), dtype=np.uint8)
    lib().orc_quant_mx_cols(R, C, _ptr(s), _ptr(q), _ptr(e))
    return q, e


def mx_scale(e8m0) -> np.ndarray:
    """E8M0 byte -> 2^(byte - 127) in fp64 (255, NaN, is never produced)."""
    return np.ldexp(1.0, np.asarray(e8m0, dtype=np.int64) - 127)


def dequant_mx_rows(q, e8m0) -> np.ndarray:
    v = e4m3_decode(q).astype(np.float64)
    return v * np.repeat(mx_scale(e8m0), MX_BLOCK, axis=1)


def dequant_mx_cols(q, e8m0) -> np.ndarray:
    v = e4m3_decode(q).astype(np.float64)
    return v * np.repeat(mx_scale(e8m0), MX_BLOCK, axis=0)


def mx_roundtrip_rows(a) -> np.ndarray:
    """Quantise rows in 1 x 32 MX blocks (from fp32) and dequantise (fp64)."""
    return dequant_mx_rows(*quant_mx_rows(np.asarray(a, dtype=np.float32)))


def mx_roundtrip_tokens(a) -> np.ndarray:
    """Quantise one expert's rows [M, C] (from fp32) in MX blocks of 32
    consecutive rows x 1 column (E8M0 scales) and dequantise (fp64): the
    operands of an MXFP8 weight-gradient product, whose contraction runs
    over the expert's rows. The blocks start at the expert's first row; the
    last one holds the M mod 32 remaining rows, quantised as the block
    zero-padded to 32 rows (zeros change neither its amax nor its kept
    codes)."""
    a = np.asarray(a, dtype=np.float32)
    M = a.shape[0]
    pad = (-M) % MX_BLOCK
    if pad:
        a = np.concatenate([a, np.zeros((pad, a.shape[1]), np.float32)])
    return dequant_mx_cols(*quant_mx_cols(a))[:M]


# ------------------------------------------------------------ expert FFN

def silu(z):
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def sigmoid64(z):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def ffn_fwd(X, W1, W2, identity: bool = False, h_fp8: bool = False, h_quant=None):
    """SwiGLU expert on rows X [M,d] (fp64): W1 [2f,d] = [gate rows; up rows],
    W2 [d,f].  G = X W1[:f]^T, U = X W1[f:]^T, H = silu(G) * U, O = H W2^T.
    With h_fp8, H is quantised per 1x128 block along f (from its fp32
    rounding) before the second product, and the dequantised H is returned;
    h_quant, when given, is the quantise-dequantise function used instead
    (MXFP8: 1 x 32 blocks).
    identity: O = X (a test mode of route/dispatch/combine)."""
    X = np.asarray(X, dtype=np.float64)
    if identity:
        return None, None, X.copy()
    W1 = np.asarray(W1, dtype=np.float64)
    W2 = np.asarray(W2, dtype=np.float64)
    f = W2.shape[1]
    GU = X @ W1.T
    H = silu(GU[:, :f]) * GU[:, f:]
    if h_fp8 and h_quant is None:
        h_quant = fp8_roundtrip_rows
    if h_quant is not None:
        H = h_quant(H.astype(np.float32))
    O = H @ W2.T
    return GU, H, O


def ffn_bwd(X, W1, W2, GU, H, dO, identity: bool = False, dgrad_fp8: bool = False,
            dgrad_quant=None, W1d=None, W2d=None, wgrad_quant=None):
    """Backward of ffn_fwd for one expert's rows (fp64).
      dH  = dO W2                    dW2 = dO^T H
      dG  = dH * U * s(G) * (1 + G (1 - s(G)))   (silu'(G) = s + G s (1 - s))
      dU  = dH * silu(G)
      dX  = [dG dU] W1               dW1 = [dG dU]^T X
    dgrad_fp8 (FP8 layers): the two data-gradient products take their
    gradient operand quantised per 1x128 block along its contraction dim
    (dO along d, [dG dU] along 2f, each from its fp32 rounding); W1, W2, X
    and H are the dequantised forward values; the weight gradients use the
    unquantised gradients. dgrad_quant, when given, replaces the 1x128
    quantise-dequantise of the gradient operands (MXFP8: 1 x 32 blocks), and
    W1d / W2d replace W1 / W2 in the two data-gradient products (MXFP8
    weights quantised in 32 x 1 blocks along those products' contraction).
    wgrad_quant, when given, is applied to every operand of the two weight-
    gradient products (dO and H for dW2, [dG dU] and X for dW1) before they
    are contracted over the expert's rows (FP8 layers: 128-row x 1 blocks,
    fp8_roundtrip_tokens); without it they take the unquantised gradients
    and the forward's (dequantised) X and H.
    Returns dX, dW1, dW2, dGU."""
    dO = np.asarray(dO, dtype=np.float64)
    if identity:
        return dO.copy(), None, None, None
    X = np.asarray(X, dtype=np.float64)
    W1 = np.asarray(W1, dtype=np.float64)
    W2 = np.asarray(W2, dtype=np.float64)
    f = W2.shape[1]
    G, U = GU[:, :f], GU[:, f:]
    if dgrad_fp8 and dgrad_quant is None:
        dgrad_quant = fp8_roundtrip_rows
    W1d = W1 if W1d is None else np.asarray(W1d, dtype=np.float64)
    W2d = W2 if W2d is None else np.asarray(W2d, dtype=np.float64)
    dOq = dgrad_quant(dO.astype(np.float32)) if dgrad_quant else dO
    dH = dOq @ W2d
    wq = wgrad_quant if wgrad_quant is not None else (lambda a: a)
    dW2 = wq(dO).T @ wq(H)
    s = sigmoid64(G)
    dG = dH * U * s * (1.0 + G * (1.0 - s))
    dU = dH * G * s
    dGU = np.concatenate([dG, dU], axis=1)
    dGUq = dgrad_quant(dGU.astype(np.float32)) if dgrad_quant else dGU
    dX = dGUq @ W1d
    dW1 = wq(dGU).T @ wq(X)
    return dX, dW1, dW2, dGU


# --------------------------------------------------------------- combine

def combine(O_perm, row_id_map, gates, O_sh=None) -> np.ndarray:
    """y[t] = sum_j g[t,j] O_perm[row_id_map[t,j]] (+ O_sh[t]), fp64."""
    O_perm = np.asarray(O_perm, dtype=np.float64)
    g = np.asarray(gates, dtype=np.float64)
    T, k = row_id_map.shape
    y = np.zeros((T, O_perm.shape[1]), dtype=np.float64)
    for j in range(k):
        y += g[:, j:j + 1] * O_perm[row_id_map[:, j]]
    if O_sh is not None:
        y += np.asarray(O_sh, dtype=np.float64)
    return y


def combine_bwd(dy, O_perm, row_id_map, gates):
    """dO_perm[row_id_map[t,j]] = g[t,j] dy[t];  dgate[t,j] = <dy[t], O_perm[row]>."""
    dy = np.asarray(dy, dtype=np.float64)
    O_perm = np.asarray(O_perm, dtype=np.float64)
    g = np.asarray(gates, dtype=np.float64)
    T, k = row_id_map.shape
    dO = np.empty((T * k, dy.shape[1]), dtype=np.float64)
    dg = np.empty((T, k), dtype=np.float64)
    for j in range(k):
        rows = row_id_map[:, j]
        dO[rows] = g[:, j:j + 1] * dy
        dg[:, j] = np.einsum("td,td->t", dy, O_perm[rows])
    return dO, dg


def dispatch_bwd(dx_perm, row_id_map, dx_add=None) -> np.ndarray:
    """dx[t] = sum_j dx_perm[row_id_map[t,j]] (+ dx_add[t])."""
    dx_perm = np.asarray(dx_perm, dtype=np.float64)
    T, k = row_id_map.shape
    dx = np.zeros((T, dx_perm.shape[1]), dtype=np.float64)
    for j in range(k):
        dx += dx_perm[row_id_map[:, j]]
    if dx_add is not None:
        dx += np.asarray(dx_add, dtype=np.float64)
    return dx


def route_bwd_logits(dgate, idx, logits, score: str, renorm: bool,
                     gate_scale: float) -> np.ndarray:
    """dL [T,E] from dgate [T,k]; selection (and any bias) is constant.
      softmax renorm : dL_e = c q_e (dg_e - sum_sel q_i dg_i), e in sel,
                       q = softmax over the selected logits
      softmax plain  : dL_e = c p_e (dg^_e - sum_sel p_i dg_i) for every e,
                       dg^_e = dg_j if e = e_j else 0
      sigmoid renorm : ds_e = c (dg_e / Z - sum_sel dg_i s_i / Z^2), e in sel
      sigmoid plain  : ds_e = c dg_e
                       dL_e = ds_e s_e (1 - s_e)."""
    L = np.asarray(logits, dtype=np.float64)
    dg = np.asarray(dgate, dtype=np.float64)
    ii = idx.astype(np.int64)
    T, E = L.shape
    c = gate_scale
    dL = np.zeros((T, E), dtype=np.float64)
    rows = np.arange(T)[:, None]
    if score == "softmax":
        if renorm:
            sel = np.take_along_axis(L, ii, axis=1)
            z = np.exp(sel - sel.max(axis=1, keepdims=True))
            q = z / z.sum(axis=1, keepdims=True)
            dsel = c * q * (dg - (q * dg).sum(axis=1, keepdims=True))
            dL[rows, ii] = dsel
        else:
            p = route_scores(L, "softmax")
            psel = np.take_along_axis(p, ii, axis=1)
            dhat = np.zeros((T, E))
            dhat[rows, ii] = dg
            dL = c * p * (dhat - (psel * dg).sum(axis=1, keepdims=True))
    else:
        sel = np.take_along_axis(L, ii, axis=1)
        s = 1.0 / (1.0 + np.exp(-sel))
        if renorm:
            Z = s.sum(axis=1, keepdims=True)
            ds = c * (dg / Z - (dg * s).sum(axis=1, keepdims=True) / (Z * Z))
        else:
            ds = c * dg
        dL[rows, ii] = ds * s * (1.0 - s)
    return dL


def route_bwd(dL, x, wr):
    """dW_r = dL^T x  [E,d];  dx_router = dL W_r  [T,d]  (fp64)."""
    X = as_f64(x)
    W = as_f64(wr)
    return dL.T @ X, dL @ W


# ------------------------------------------ load-balancing auxiliary loss

def aux_loss(logits, idx, E: int, coeff: float) -> float:
    """Load-balancing auxiliary loss, Switch-Transformer form (the pages name
    the loss and its 0.01 coefficient, skill page workflow "Fluxo 2"; they give
    no formula, and routing fuses it, Megatron Core MoE summary section 2.4):
      f_e  = #{(t, j): idx[t,j] = e} / (T k)      share of the routing slots
      P_e  = (1/T) sum_t softmax(L[t,:])_e       mean router probability
      loss = coeff * E * sum_e f_e P_e
    The probabilities are the softmax over all experts whatever the gate's
    score function; f is a constant of the routing (no gradient). fp64."""
    L = np.asarray(logits, dtype=np.float64)
    T = L.shape[0]
    k = np.asarray(idx).shape[1]
    p = np.exp(L - L.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    f = np.bincount(np.asarray(idx, dtype=np.int64).reshape(-1), minlength=E) / float(T * k)
    return float(coeff * E * np.dot(f, p.mean(axis=0)))


def aux_loss_dlogits(logits, idx, E: int, coeff: float, d_aux: float = 1.0) -> np.ndarray:
    """d(aux_loss)/dL [T,E] times the upstream gradient d_aux (fp64):
    coeff * E / T * d_aux * p[t,e] * (f_e - sum_j f_j p[t,j])."""
    L = np.asarray(logits, dtype=np.float64)
    T = L.shape[0]
    k = np.asarray(idx).shape[1]
    p = np.exp(L - L.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    f = np.bincount(np.asarray(idx, dtype=np.int64).reshape(-1), minlength=E) / float(T * k)
    return coeff * E / T * d_aux * p * (f[None, :] - (p @ f)[:, None])


# -------------------------------------------------------- the whole layer

# 8-bit layers: whether the weight-gradient operands are quantised in token
# blocks inside each expert's rows (FP8: 128-row x 1 blocks with fp32 scales,
# fp8_roundtrip_tokens; MXFP8: 32-row x 1 blocks with E8M0 scales,
# mx_roundtrip_tokens) or taken unquantised (the forward's dequantised X and
# H, the bf16 gradients)
FP8_WGRAD_TOKEN_BLOCKS = True
MXFP8_WGRAD_TOKEN_BLOCKS = True


def _expert_weight(w, e):
    """Expert e's weight from a stacked [E, ...] array/tensor or a callable."""
    return w(e) if callable(w) else w[e]


def layer_stream(cfg, inp: dict, identity: bool = False, on_expert=None,
                 fp8_wgrad: Optional[bool] = None) -> dict:
    """Forward and backward of one MoE layer on the CPU, one expert at a
    time, so that no tensor with an expert dimension is ever held whole.

    inp: x [T,d], wr [E,d], bias [E] or None, dy [T,d], w1 and w2 (a stacked
    [E,2f,d] / [E,d,f] array or tensor, or a callable e -> that expert's
    weight), sw1/sw2 (shared expert, when cfg.shared); torch or numpy.
    For fp8 weights the oracle quantises the bf16 masters itself in
    128 x 128 blocks and the dispatched rows per 1 x 128 block; H, dO and
    [dG dU] are quantised per 1 x 128 before the product that contracts them
    along their rows (ffn_fwd, ffn_bwd); with fp8_wgrad (default:
    FP8_WGRAD_TOKEN_BLOCKS, MXFP8_WGRAD_TOKEN_BLOCKS) the four operands of the weight-gradient products are
    quantised in 128-row x 1 blocks inside each expert's rows
    (fp8_roundtrip_tokens). For mxfp8 every operand of the six expert
    products is quantised in blocks of 32 along that product's contraction
    dimension with E8M0 scales: x, H, dO and [dG dU] in 1 x 32 row blocks
    for the forward and data-gradient products; W1 and W2 in row blocks for
    the forward and in 32 x 1 column blocks for the data gradients; with
    fp8_wgrad the four operands of the weight-gradient products (the
    dequantised x and H, the unquantised dO and [dG dU]) in 32-row x 1
    blocks inside each expert's rows (mx_roundtrip_tokens); without it the
    weight gradients take those four unquantised.

    on_expert(e, r0, r1, t), when given, is called for every expert in order
    with its rows [r0, r1) of the dispatched order and t = dict(out_perm,
    act_gu, act_h, d_out_perm, dx_perm (those rows), dw1, dw2, w_q (the
    quantised weights, FP8 layers)), or t = None for an expert with no rows
    (its weight gradients are zero). The returned dict holds every tensor
    without an expert dimension.
    """
    E, k, f = cfg.E, cfg.k, cfg.f
    mx = cfg.weight == "mxfp8"
    fp8 = cfg.weight == "fp8"
    if fp8_wgrad is None:
        fp8_wgrad = (fp8 and FP8_WGRAD_TOKEN_BLOCKS) or (mx and MXFP8_WGRAD_TOKEN_BLOCKS)
    qb = cfg.quant_block
    h_quant = mx_roundtrip_rows if mx else (fp8_roundtrip_rows if fp8 else None)
    w_quant = None
    if fp8_wgrad and fp8:
        w_quant = fp8_roundtrip_tokens
    elif fp8_wgrad and mx:
        w_quant = mx_roundtrip_tokens
    out = {}
    L, idx, g = route(cfg, inp["x"], inp["wr"], inp.get("bias"))
    out.update(logits=L, idx=idx, gates=g)
    counts, offsets, rmap, ptok = dispatch_index(idx, E)
    out.update(counts=counts, offsets=offsets, row_id_map=rmap, perm_token=ptok)
    T, d = cfg.T, cfg.d
    x32 = as_f32(inp["x"])
    # the dispatched rows' values (dequantised for FP8 layers), per token
    if mx:
        xq, xs = quant_mx_rows(x32)
        out.update(xq=xq, x_scale=xs)
        Xt = dequant_mx_rows(xq, xs)
    elif fp8:
        xq, xs = quant_blocks(x32, 1, qb)
        out.update(xq=xq, x_scale=xs)
        Xt = dequant_blocks(xq, xs, 1, qb)
    else:
        Xt = x32.astype(np.float64)

    def expert_weights(w1, w2):
        w1 = as_f32(w1)
        w2 = as_f32(w2)
        if mx:
            r1, r2 = quant_mx_rows(w1), quant_mx_rows(w2)
            c1, c2 = quant_mx_cols(w1), quant_mx_cols(w2)
            return (dequant_mx_rows(*r1), dequant_mx_rows(*r2),
                    dict(w1_rows=r1, w2_rows=r2, w1_cols=c1, w2_cols=c2,
                         W1d=dequant_mx_cols(*c1), W2d=dequant_mx_cols(*c2)))
        if not fp8:
            return w1.astype(np.float64), w2.astype(np.float64), None
        q1, s1 = quant_blocks(w1, qb, qb)
        q2, s2 = quant_blocks(w2, qb, qb)
        return (dequant_blocks(q1, s1, qb, qb), dequant_blocks(q2, s2, qb, qb),
                (q1, s1, q2, s2))

    dy = as_f64(inp["dy"])
    # gate and slot of every dispatched row
    gate_row = np.empty(T * k)
    slot_row = np.empty(T * k, dtype=np.int64)
    gate_row[rmap.reshape(-1)] = np.asarray(g, np.float64).reshape(-1)
    slot_row[rmap.reshape(-1)] = np.tile(np.arange(k), T)
    y = np.zeros((T, d))
    dgate = np.zeros((T, k))
    dx = np.zeros((T, d))
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            if on_expert:
                on_expert(e, r0, r1, None)
            continue
        toks = ptok[r0:r1]          # distinct tokens: one row per token and expert
        Xe = Xt[toks]
        if identity:
            W1 = W2 = wq = None
        else:
            W1, W2, wq = expert_weights(_expert_weight(inp["w1"], e), _expert_weight(inp["w2"], e))
        gu, h, o = ffn_fwd(Xe, W1, W2, identity, h_quant=h_quant)
        ge = gate_row[r0:r1, None]
        y[toks] += ge * o                                      # combine
        dgate[toks, slot_row[r0:r1]] = np.einsum("rd,rd->r", dy[toks], o)
        dOe = ge * dy[toks]                                    # combine backward
        dxe, dw1, dw2, _ = ffn_bwd(Xe, W1, W2, gu, h, dOe, identity, dgrad_quant=h_quant,
                                   W1d=wq["W1d"] if mx else None, W2d=wq["W2d"] if mx else None,
                                   wgrad_quant=w_quant)
        dx[toks] += dxe                                        # dispatch backward
        if on_expert:
            on_expert(e, r0, r1, dict(out_perm=o, act_gu=gu, act_h=h, d_out_perm=dOe, dx_perm=dxe,
                                      dw1=dw1, dw2=dw2, w_q=wq))
    if cfg.shared:
        SW1, SW2, sq = (None, None, None) if identity else expert_weights(inp["sw1"], inp["sw2"])
        sgu, sh, O_sh = ffn_fwd(Xt, SW1, SW2, identity, h_quant=h_quant)
        out.update(shared_out=O_sh, shared_gu=sgu, shared_h=sh)
        y += O_sh
        dx_sh, sdw1, sdw2, _ = ffn_bwd(Xt, SW1, SW2, sgu, sh, dy, identity, dgrad_quant=h_quant,
                                       W1d=sq["W1d"] if mx else None,
                                       W2d=sq["W2d"] if mx else None, wgrad_quant=w_quant)
        out.update(shared_dx=dx_sh, shared_dw1=sdw1, shared_dw2=sdw2)
        if fp8 or mx:
            out["shared_w_q"] = sq
        dx += dx_sh
    out.update(y=y, d_gate=dgate)
    dL = route_bwd_logits(dgate, idx, L, cfg.score, cfg.renorm, cfg.gate_scale)
    if cfg.aux_coeff:
        # the auxiliary loss enters the step's total loss with weight 1
        out["aux_loss"] = aux_loss(L, idx, E, cfg.aux_coeff)
        dL = dL + aux_loss_dlogits(L, idx, E, cfg.aux_coeff, 1.0)
    dWr, dx_r = route_bwd(dL, inp["x"], inp["wr"])
    out.update(d_logits=dL, dw_router=dWr, dx=dx + dx_r, dx_router=dx_r)
    return out


def layer(cfg, inp: dict, identity: bool = False, fp8_wgrad: Optional[bool] = None) -> dict:
    """Forward and backward of one MoE layer on the CPU, every tensor
    (layer_stream, with the per-expert tensors gathered): x_perm (or the FP8
    codes and scales xq_perm, x_scale_perm), out_perm, act_gu, act_h,
    d_out_perm, dx_perm [A, ...] in dispatched order; dw1 [E,2f,d], dw2
    [E,d,f]; w_q, each expert's quantised weights (FP8 layers); and every
    tensor layer_stream returns. For small layers (it holds everything)."""
    E, f, d, A = cfg.E, cfg.f, cfg.d, cfg.T * cfg.k
    full = dict(out_perm=np.zeros((A, d)), act_gu=np.zeros((A, 2 * f)), act_h=np.zeros((A, f)),
                d_out_perm=np.zeros((A, d)), dx_perm=np.zeros((A, d)),
                dw1=np.zeros((E, 2 * f, d)), dw2=np.zeros((E, d, f)))
    w_q = [None] * E

    def keep(e, r0, r1, t):
        if t is None:
            return
        for n in ("out_perm", "d_out_perm", "dx_perm"):
            full[n][r0:r1] = t[n]
        if not identity:
            for n in ("act_gu", "act_h"):
                full[n][r0:r1] = t[n]
            full["dw1"][e] = t["dw1"]
            full["dw2"][e] = t["dw2"]
        w_q[e] = t["w_q"]

    out = layer_stream(cfg, inp, identity, on_expert=keep, fp8_wgrad=fp8_wgrad)
    rmap = out["row_id_map"]
    if "xq" in out:
        out.update(xq_perm=permute(out["xq"], rmap), x_scale_perm=permute(out["x_scale"], rmap))
    else:
        out["x_perm"] = permute(as_f32(inp["x"]), rmap)
    out.update(full)
    if cfg.weight in ("fp8", "mxfp8"):
        out["w_q"] = w_q
    return out


def rel_l2(a, b) -> float:
    """||a - b||_2 / ||b||_2 (b is the oracle), in fp64."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b.ravel())
    na = np.linalg.norm((a - b).ravel())
    if nb == 0.0:
        return 0.0 if na == 0.0 else float("inf")
    return float(na / nb)
