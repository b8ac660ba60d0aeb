"""ctypes binding of libmoe.so (the C ABI in include/moe.h).

Argument marshalling only: every step of the layer runs in the library's
HIP kernels. Tensors are torch tensors on the GPU (PyTorch provides device
memory and the current stream); pointers, sizes and the stream handle are
passed through unchanged. A missing library is an error: there is no
fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

MOE_OK = 0
STATUS = {0: "MOE_OK", -1: "MOE_ERR_INVALID_ARG", -2: "MOE_ERR_UNSUPPORTED_DTYPE",
          -3: "MOE_ERR_ALIGNMENT", -4: "MOE_ERR_WORKSPACE", -5: "MOE_ERR_HIP"}
DTYPE = {"f32": 0, "bf16": 1, "fp8": 2, "mxfp8": 3}
SCORE = {"softmax": 0, "sigmoid": 1}
GROUP_SCORE = {"top2_sum": 0, "max": 1}
OP_ROUTE, OP_DISPATCH, OP_GROUPED_FFN, OP_GROUPED_FFN_BWD, OP_ROUTE_BWD, OP_AUX_LOSS = range(6)

EXPORTS = ["moe_workspace_size", "moe_route", "moe_dispatch", "moe_route_dispatch", "moe_dispatch_scratch",
           "moe_grouped_ffn", "moe_combine",
           "moe_combine_bwd", "moe_grouped_ffn_bwd", "moe_dispatch_bwd", "moe_route_bwd",
           "moe_route_aux_loss",
           "moe_quantize_fp8_blockwise", "moe_quantize_mxfp8", "moe_status_string"]


class MoeError(RuntimeError):
    def __init__(self, name, rc):
        super().__init__(f"{name} failed: {STATUS.get(rc, rc)}")
        self.rc = rc


class MoeConfig(ctypes.Structure):
    _fields_ = [
        ("num_tokens", ctypes.c_int64),
        ("hidden", ctypes.c_int64),
        ("num_experts", ctypes.c_int64),
        ("top_k", ctypes.c_int64),
        ("ffn_hidden", ctypes.c_int64),
        ("score_fn", ctypes.c_int32),
        ("renormalize", ctypes.c_int32),
        ("gate_scale", ctypes.c_float),
        ("num_groups", ctypes.c_int32),
        ("topk_groups", ctypes.c_int32),
        ("group_score", ctypes.c_int32),
        ("act_dtype", ctypes.c_int32),
        ("weight_dtype", ctypes.c_int32),
        ("quant_block", ctypes.c_int32),
        ("ffn_mode", ctypes.c_int32),
        ("gemm_tile", ctypes.c_int32),
        ("aux_coeff", ctypes.c_float),
        ("recompute", ctypes.c_int32),
    ]

TILE = {"auto": 0, "small": 1, "big": 2}
RECOMPUTE = {"none": 0, "act": 1, "full": 2}


def make_config(T, d, E, k, f, score="softmax", renorm=True, gate_scale=1.0, num_groups=1,
                topk_groups=1, group_score="top2_sum", act="bf16", weight="bf16",
                quant_block=128, identity=False, gemm_tile="auto", aux_coeff=0.0,
                recompute="none", **_ignored) -> MoeConfig:
    return MoeConfig(T, d, E, k, f, SCORE[score], int(bool(renorm)), float(gate_scale),
                     num_groups, topk_groups, GROUP_SCORE[group_score], DTYPE[act], DTYPE[weight],
                     quant_block, 1 if identity else 0, TILE[gemm_tile], float(aux_coeff),
                     RECOMPUTE[recompute])


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        C = ctypes.POINTER(MoeConfig)
        sz = ctypes.c_size_t
        i64 = ctypes.c_int64
        sig = {
            "moe_workspace_size": (sz, [C, ctypes.c_int]),
            "moe_route": (ctypes.c_int, [C, P, P, P, P, P, P, P, P, sz, P]),
            "moe_dispatch": (ctypes.c_int, [C, P, P, P, P, P, P, P, P, P, sz, P]),
            "moe_route_dispatch": (ctypes.c_int, [C] + [P] * 14 + [sz, P]),
            "moe_dispatch_scratch": (ctypes.c_int, [C, P, P, P, P, P, P, P, P, P]),
            "moe_grouped_ffn": (ctypes.c_int, [C, P, P, P, P, P, P, P, P, P, P, P, P, sz, P]),
            "moe_combine": (ctypes.c_int, [C, P, P, P, P, P, P]),
            "moe_combine_bwd": (ctypes.c_int, [C, P, P, P, P, P, P, P]),
            "moe_grouped_ffn_bwd": (ctypes.c_int, [C] + [P] * 15 + [sz, P]),
            "moe_dispatch_bwd": (ctypes.c_int, [C, P, P, P, P, P]),
            "moe_route_bwd": (ctypes.c_int, [C] + [P] * 10 + [sz, P]),
            "moe_route_aux_loss": (ctypes.c_int, [C, P, P, P, P, sz, P]),
            "moe_quantize_fp8_blockwise": (ctypes.c_int, [P, ctypes.c_int, i64, i64, i64, i64, P, P, P]),
            "moe_quantize_mxfp8": (ctypes.c_int, [P, ctypes.c_int, i64, i64, ctypes.c_int, P, P, P]),
            "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _p(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def _check(name, rc):
    if rc != MOE_OK:
        raise MoeError(name, rc)


def workspace_size(cfg: MoeConfig, op: int) -> int:
    return lib().moe_workspace_size(ctypes.byref(cfg), op)


def moe_route(cfg, x, w_router, expert_bias, logits, topk_idx, topk_gate, routing_map=None,
              ws=None, stream=None):
    _check("moe_route", lib().moe_route(ctypes.byref(cfg), _p(x), _p(w_router), _p(expert_bias),
                                        _p(logits), _p(topk_idx), _p(topk_gate), _p(routing_map),
                                        _p(ws), _nbytes(ws), _stream(stream)))


def moe_dispatch(cfg, x, topk_idx, counts, offsets, row_id_map, perm_token, x_perm, x_scale=None,
                 ws=None, stream=None):
    _check("moe_dispatch", lib().moe_dispatch(ctypes.byref(cfg), _p(x), _p(topk_idx), _p(counts),
                                              _p(offsets), _p(row_id_map), _p(perm_token),
                                              _p(x_perm), _p(x_scale), _p(ws), _nbytes(ws),
                                              _stream(stream)))


def moe_route_dispatch(cfg, x, w_router, expert_bias, logits, topk_idx, topk_gate, routing_map,
                       counts, offsets, row_id_map, perm_token, x_perm, x_scale=None, ws=None,
                       stream=None):
    _check("moe_route_dispatch", lib().moe_route_dispatch(
        ctypes.byref(cfg), _p(x), _p(w_router), _p(expert_bias), _p(logits), _p(topk_idx),
        _p(topk_gate), _p(routing_map), _p(counts), _p(offsets), _p(row_id_map), _p(perm_token),
        _p(x_perm), _p(x_scale), _p(ws), _nbytes(ws), _stream(stream)))


def moe_dispatch_scratch(cfg, x, topk_idx, counts, offsets, row_id_map, perm_token, x_perm,
                         x_scale=None, stream=None):
    _check("moe_dispatch_scratch", lib().moe_dispatch_scratch(
        ctypes.byref(cfg), _p(x), _p(topk_idx), _p(counts), _p(offsets), _p(row_id_map),
        _p(perm_token), _p(x_perm), _p(x_scale), _stream(stream)))


def moe_grouped_ffn(cfg, x_perm, x_scale, offsets, w1, w1_scale, w2, w2_scale, act_gu, act_h,
                    h_scale, out_perm, ws=None, stream=None):
    _check("moe_grouped_ffn", lib().moe_grouped_ffn(
        ctypes.byref(cfg), _p(x_perm), _p(x_scale), _p(offsets), _p(w1), _p(w1_scale), _p(w2),
        _p(w2_scale), _p(act_gu), _p(act_h), _p(h_scale), _p(out_perm), _p(ws), _nbytes(ws),
        _stream(stream)))


def moe_combine(cfg, out_perm, row_id_map, topk_gate, shared_out, y, stream=None):
    _check("moe_combine", lib().moe_combine(ctypes.byref(cfg), _p(out_perm), _p(row_id_map),
                                            _p(topk_gate), _p(shared_out), _p(y), _stream(stream)))


def moe_combine_bwd(cfg, dy, out_perm, row_id_map, topk_gate, d_out_perm, d_gate, stream=None):
    _check("moe_combine_bwd", lib().moe_combine_bwd(ctypes.byref(cfg), _p(dy), _p(out_perm),
                                                    _p(row_id_map), _p(topk_gate), _p(d_out_perm),
                                                    _p(d_gate), _stream(stream)))


def moe_grouped_ffn_bwd(cfg, x_perm, x_scale, offsets, w1, w1_scale, w2, w2_scale, act_gu, act_h,
                        h_scale, d_out_perm, dx_perm, dw1, dw2, ws=None, stream=None):
    _check("moe_grouped_ffn_bwd", lib().moe_grouped_ffn_bwd(
        ctypes.byref(cfg), _p(x_perm), _p(x_scale), _p(offsets), _p(w1), _p(w1_scale), _p(w2),
        _p(w2_scale), _p(act_gu), _p(act_h), _p(h_scale), _p(d_out_perm), _p(dx_perm), _p(dw1),
        _p(dw2), _p(ws), _nbytes(ws), _stream(stream)))


def moe_dispatch_bwd(cfg, dx_perm, row_id_map, dx_add, dx, stream=None):
    _check("moe_dispatch_bwd", lib().moe_dispatch_bwd(ctypes.byref(cfg), _p(dx_perm),
                                                      _p(row_id_map), _p(dx_add), _p(dx),
                                                      _stream(stream)))


def moe_route_aux_loss(cfg, logits, topk_idx, aux_loss, ws=None, stream=None):
    _check("moe_route_aux_loss", lib().moe_route_aux_loss(ctypes.byref(cfg), _p(logits),
                                                          _p(topk_idx), _p(aux_loss), _p(ws),
                                                          _nbytes(ws), _stream(stream)))


def moe_route_bwd(cfg, x, w_router, logits, topk_idx, topk_gate, d_gate, dx, dw_router, ws=None,
                  stream=None, d_aux=None):
    _check("moe_route_bwd", lib().moe_route_bwd(ctypes.byref(cfg), _p(x), _p(w_router), _p(logits),
                                                _p(topk_idx), _p(topk_gate), _p(d_gate), _p(d_aux),
                                                _p(dx), _p(dw_router), _p(ws), _nbytes(ws),
                                                _stream(stream)))


def moe_quantize_fp8_blockwise(src, rows, cols, block_r, block_c, dst, scale, stream=None):
    import torch
    sdt = {torch.float32: 0, torch.bfloat16: 1}[src.dtype]
    _check("moe_quantize_fp8_blockwise", lib().moe_quantize_fp8_blockwise(
        _p(src), sdt, rows, cols, block_r, block_c, _p(dst), _p(scale), _stream(stream)))


def moe_quantize_mxfp8(src, rows, cols, colwise, dst, e8m0, stream=None):
    import torch
    sdt = {torch.float32: 0, torch.bfloat16: 1}[src.dtype]
    _check("moe_quantize_mxfp8", lib().moe_quantize_mxfp8(
        _p(src), sdt, rows, cols, int(bool(colwise)), _p(dst), _p(e8m0), _stream(stream)))


def moe_status_string(rc: int) -> str:
    return lib().moe_status_string(rc).decode()
