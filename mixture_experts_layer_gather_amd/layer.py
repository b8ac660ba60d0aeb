"""One MoE layer's token path on one GPU, driven through libmoe.

Buffers are allocated once, at construction, with sizes that follow from the
configuration alone (dropless: exactly T*k dispatched rows), so the forward
and backward passes never synchronise with the host to size a tensor
(Hybrid-EP article, buffer pre-allocation paragraph; Megatron Core MoE
summary, section 2.4, device-initiated kernels). Every stage is one or more
libmoe calls on the current stream.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _lib as L

_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16}


class MoELayer:
    def __init__(self, T, d, E, k, f, shared=0, score="softmax", renorm=True, gate_scale=1.0,
                 num_groups=1, topk_groups=1, group_score="top2_sum", act="bf16", weight="bf16",
                 quant_block=128, identity=False, gemm_tile="auto", aux_coeff=0.0, recompute="none",
                 device="cuda", **_ignored):
        self.T, self.d, self.E, self.k, self.f = T, d, E, k, f
        self.A = T * k
        self.shared = int(shared)
        self.act, self.weight = act, weight
        self.mx = weight == "mxfp8"
        self.fp8 = weight in ("fp8", "mxfp8")   # E4M3 codes, with either scale kind
        self.qb = quant_block
        # scales: fp32 per 1 x 128 / 128 x 128 block, or E8M0 bytes per 32
        sdt = torch.uint8 if self.mx else torch.float32
        kw = dict(score=score, renorm=renorm, gate_scale=gate_scale, num_groups=num_groups,
                  topk_groups=topk_groups, group_score=group_score, act=act, weight=weight,
                  quant_block=quant_block, identity=identity, gemm_tile=gemm_tile,
                  aux_coeff=aux_coeff, recompute=recompute)
        self.cfg = L.make_config(T, d, E, k, f, **kw)
        self.aux = aux_coeff != 0.0
        self.scfg = L.make_config(T, d, 1, 1, f, act=act, weight=weight, quant_block=quant_block,
                                  identity=identity, gemm_tile=gemm_tile, recompute=recompute)
        # activations the expert FFN keeps from forward to backward: GU and H,
        # GU only ("act": H is rebuilt from it), or nothing ("full")
        keep_gu = recompute != "full"
        keep_h = recompute == "none"
        dev = torch.device(device)
        at = _TORCH[act]
        pt = torch.float32 if weight == "f32" else torch.bfloat16   # parameter dtype
        self.param_dtype = pt
        A = self.A
        e = lambda *s, dt=at: torch.empty(*s, dtype=dt, device=dev)
        i32 = torch.int32
        # routing
        self.logits = e(T, E, dt=torch.float32)
        self.topk_idx = e(T, k, dt=i32)
        self.topk_gate = e(T, k, dt=torch.float32)
        self.routing_map = e(T, E, dt=torch.uint8)
        # auxiliary loss: its value, and its weight in the step's total loss
        # (1, the upstream gradient of the backward)
        self.aux_loss = e(1, dt=torch.float32)
        self.d_aux = torch.ones(1, dtype=torch.float32, device=dev)
        # dispatch
        self.counts = e(E, dt=i32)
        self.offsets = e(E + 1, dt=i32)
        self.row_id_map = e(T, k, dt=i32)
        self.perm_token = e(A, dt=i32)
        self.act_h = self.h_scale = None
        if self.fp8:
            self.x_perm = e(A, d, dt=torch.uint8)
            self.x_scale = e(A, d // quant_block, dt=sdt)
            if keep_h:
                self.act_h = e(A, f, dt=torch.uint8)
                self.h_scale = e(A, f // quant_block, dt=sdt)
        else:
            self.x_perm = e(A, d)
            self.x_scale = None
            if keep_h:
                self.act_h = e(A, f)
        self.act_gu = e(A, 2 * f) if keep_gu else None
        self.out_perm = e(A, d)
        self.y = e(T, d)
        # backward
        self.d_out_perm = e(A, d)
        self.d_gate = e(T, k, dt=torch.float32)
        self.dx_perm = e(A, d)
        self.dx = e(T, d)
        self.dw1 = e(E, 2 * f, d, dt=pt)
        self.dw2 = e(E, d, f, dt=pt)
        self.dw_router = e(E, d, dt=torch.float32)
        # workspaces
        u8 = torch.uint8
        self.ws_dispatch = e(max(1, L.workspace_size(self.cfg, L.OP_DISPATCH)), dt=u8)
        self.ws_ffn = e(max(1, L.workspace_size(self.cfg, L.OP_GROUPED_FFN),
                            L.workspace_size(self.scfg, L.OP_GROUPED_FFN)), dt=u8)
        self.ws_ffn_bwd = e(max(1, L.workspace_size(self.cfg, L.OP_GROUPED_FFN_BWD),
                                L.workspace_size(self.scfg, L.OP_GROUPED_FFN_BWD)), dt=u8)
        self.ws_route_bwd = e(max(1, L.workspace_size(self.cfg, L.OP_ROUTE_BWD)), dt=u8)
        self.ws_aux = e(max(1, L.workspace_size(self.cfg, L.OP_AUX_LOSS)), dt=u8)
        if self.shared:
            self.s_offsets = torch.tensor([0, T], dtype=i32, device=dev)
            self.s_h = self.s_h_scale = None
            if self.fp8:
                self.s_x = e(T, d, dt=torch.uint8)
                self.s_x_scale = e(T, d // quant_block, dt=sdt)
                if keep_h:
                    self.s_h = e(T, f, dt=torch.uint8)
                    self.s_h_scale = e(T, f // quant_block, dt=sdt)
            elif keep_h:
                self.s_h = e(T, f)
            self.s_gu = e(T, 2 * f) if keep_gu else None
            self.s_out = e(T, d)
            self.s_dx = e(T, d)
            self.s_dw1 = e(1, 2 * f, d, dt=pt)
            self.s_dw2 = e(1, d, f, dt=pt)
        self.x = None

    # ------------------------------------------------------------ weights
    def _quant_weight(self, w):
        """128 x 128 block FP8 of an expert weight stack [G, R, C] (setup step)."""
        G, R, C = w.shape
        qb = self.qb
        q = torch.empty(G, R, C, dtype=torch.uint8, device=w.device)
        s = torch.empty(G, R // qb, C // qb, dtype=torch.float32, device=w.device)
        L.moe_quantize_fp8_blockwise(w, G * R, C, qb, qb, q, s)
        return q, s

    def _quant_weight_mx(self, w, colwise):
        """MXFP8 of an expert weight stack [G, R, C] (setup step): 1 x 32
        blocks along C (rows) for the forward products, 32 x 1 blocks along
        R (columns) for the data-gradient products; R is a multiple of 32,
        so no block spans two experts."""
        G, R, C = w.shape
        q = torch.empty(G, R, C, dtype=torch.uint8, device=w.device)
        s = torch.empty(G, R // 32, C, dtype=torch.uint8, device=w.device) if colwise else \
            torch.empty(G, R, C // 32, dtype=torch.uint8, device=w.device)
        L.moe_quantize_mxfp8(w, G * R, C, colwise, q, s)
        return q, s

    def set_weights(self, w_router, w1, w2, bias=None, sw1=None, sw2=None):
        self.w_router = w_router
        self.bias = bias
        self.w1_master, self.w2_master = w1, w2
        # the weights the backward's data-gradient products read (MXFP8:
        # column-quantised copies; otherwise the forward's)
        if self.mx:
            self.w1, self.w1_scale = self._quant_weight_mx(w1, False)
            self.w2, self.w2_scale = self._quant_weight_mx(w2, False)
            self.w1b, self.w1b_scale = self._quant_weight_mx(w1, True)
            self.w2b, self.w2b_scale = self._quant_weight_mx(w2, True)
        elif self.fp8:
            self.w1, self.w1_scale = self._quant_weight(w1)
            self.w2, self.w2_scale = self._quant_weight(w2)
        else:
            self.w1, self.w2 = w1, w2
            self.w1_scale = self.w2_scale = None
        if not self.mx:
            self.w1b, self.w1b_scale, self.w2b, self.w2b_scale = self.w1, self.w1_scale, self.w2, self.w2_scale
        if self.shared:
            sw1 = sw1.reshape(1, *sw1.shape[-2:])
            sw2 = sw2.reshape(1, *sw2.shape[-2:])
            if self.mx:
                self.sw1, self.sw1_scale = self._quant_weight_mx(sw1, False)
                self.sw2, self.sw2_scale = self._quant_weight_mx(sw2, False)
                self.sw1b, self.sw1b_scale = self._quant_weight_mx(sw1, True)
                self.sw2b, self.sw2b_scale = self._quant_weight_mx(sw2, True)
            elif self.fp8:
                self.sw1, self.sw1_scale = self._quant_weight(sw1)
                self.sw2, self.sw2_scale = self._quant_weight(sw2)
            else:
                self.sw1, self.sw2 = sw1, sw2
                self.sw1_scale = self.sw2_scale = None
            if not self.mx:
                self.sw1b, self.sw1b_scale = self.sw1, self.sw1_scale
                self.sw2b, self.sw2b_scale = self.sw2, self.sw2_scale

    def quantize_shared_input(self, x):
        """The shared expert's input in the layer's FP8 format (its rows are
        the unpermuted tokens)."""
        if self.mx:
            L.moe_quantize_mxfp8(x, self.T, self.d, False, self.s_x, self.s_x_scale)
        else:
            L.moe_quantize_fp8_blockwise(x, self.T, self.d, 1, self.qb, self.s_x, self.s_x_scale)

    # ------------------------------------------------------------ passes
    def _shared_fwd(self, x):
        sx, sxs = x, None
        if self.fp8:
            self.quantize_shared_input(x)
            sx, sxs = self.s_x, self.s_x_scale
        L.moe_grouped_ffn(self.scfg, sx, sxs, self.s_offsets, self.sw1, self.sw1_scale,
                          self.sw2, self.sw2_scale, self.s_gu, self.s_h, self.s_h_scale,
                          self.s_out, self.ws_ffn)

    def _shared_bwd(self, dy):
        sx, sxs = (self.s_x, self.s_x_scale) if self.fp8 else (self.x, None)
        L.moe_grouped_ffn_bwd(self.scfg, sx, sxs, self.s_offsets, self.sw1b, self.sw1b_scale,
                              self.sw2b, self.sw2b_scale, self.s_gu, self.s_h, self.s_h_scale,
                              dy, self.s_dx, self.s_dw1, self.s_dw2, self.ws_ffn_bwd)

    def forward(self, x: torch.Tensor, mark=None) -> torch.Tensor:
        """mark(name), when given, is called after each library call (the
        benchmark records an event on the current stream there)."""
        mark = mark or (lambda name: None)
        self.x = x
        c = self.cfg
        L.moe_route(c, x, self.w_router, self.bias, self.logits, self.topk_idx, self.topk_gate,
                    self.routing_map)
        mark("route")
        if self.aux:
            L.moe_route_aux_loss(c, self.logits, self.topk_idx, self.aux_loss, self.ws_aux)
            mark("aux_loss")
        L.moe_dispatch(c, x, self.topk_idx, self.counts, self.offsets, self.row_id_map,
                       self.perm_token, self.x_perm, self.x_scale, self.ws_dispatch)
        mark("dispatch")
        L.moe_grouped_ffn(c, self.x_perm, self.x_scale, self.offsets, self.w1, self.w1_scale,
                          self.w2, self.w2_scale, self.act_gu, self.act_h, self.h_scale,
                          self.out_perm, self.ws_ffn)
        mark("grouped_ffn")
        shared_out = None
        if self.shared:
            self._shared_fwd(x)
            mark("shared_ffn")
            shared_out = self.s_out
        L.moe_combine(c, self.out_perm, self.row_id_map, self.topk_gate, shared_out, self.y)
        mark("combine")
        return self.y

    def backward(self, dy: torch.Tensor, mark=None) -> torch.Tensor:
        mark = mark or (lambda name: None)
        c = self.cfg
        L.moe_combine_bwd(c, dy, self.out_perm, self.row_id_map, self.topk_gate, self.d_out_perm,
                          self.d_gate)
        mark("combine_bwd")
        L.moe_grouped_ffn_bwd(c, self.x_perm, self.x_scale, self.offsets, self.w1b, self.w1b_scale,
                              self.w2b, self.w2b_scale, self.act_gu, self.act_h, self.h_scale,
                              self.d_out_perm, self.dx_perm, self.dw1, self.dw2, self.ws_ffn_bwd)
        mark("grouped_ffn_bwd")
        dx_add = None
        if self.shared:
            self._shared_bwd(dy)
            mark("shared_ffn_bwd")
            dx_add = self.s_dx
        L.moe_dispatch_bwd(c, self.dx_perm, self.row_id_map, dx_add, self.dx)
        mark("dispatch_bwd")
        L.moe_route_bwd(c, self.x, self.w_router, self.logits, self.topk_idx, self.topk_gate,
                        self.d_gate, self.dx, self.dw_router, self.ws_route_bwd,
                        d_aux=self.d_aux if self.aux else None)
        mark("route_bwd")
        return self.dx

    def step(self, x, dy):
        """One forward and backward pass of the layer."""
        self.forward(x)
        return self.backward(dy)
