"""MI355X-native MoE layer token path: route -> dispatch -> grouped SwiGLU
expert GEMMs -> combine, forward and backward, as hand-written HIP kernels for
gfx950 behind the C ABI in include/moe.h (libmoe.so, built in-tree)."""
from ._lib import (MoeConfig, MoeError, make_config, workspace_size, lib, moe_route, moe_dispatch,
                   moe_route_dispatch, moe_dispatch_scratch, moe_grouped_ffn, moe_combine, moe_combine_bwd, moe_grouped_ffn_bwd,
                   moe_dispatch_bwd, moe_route_bwd, moe_quantize_fp8_blockwise, moe_quantize_mxfp8, moe_status_string,
                   EXPORTS, LIB_PATH, RECOMPUTE)
from .layer import MoELayer

__all__ = ["MoeConfig", "MoeError", "make_config", "workspace_size", "lib", "moe_route",
           "moe_dispatch", "moe_route_dispatch", "moe_dispatch_scratch", "moe_grouped_ffn", "moe_combine", "moe_combine_bwd",
           "moe_grouped_ffn_bwd", "moe_dispatch_bwd", "moe_route_bwd",
           "moe_quantize_fp8_blockwise", "moe_quantize_mxfp8", "moe_status_string", "MoELayer", "EXPORTS", "LIB_PATH", "RECOMPUTE"]
