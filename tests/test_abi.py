"""Host-side tests of the C ABI (no GPU needed): the library loads, exports
every function include/moe.h declares, sizes workspaces from the config alone
and rejects bad arguments before enqueueing anything."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def M():
    import mixture_experts_layer_gather_amd as m
    if not os.path.exists(m.LIB_PATH):
        from mixture_experts_layer_gather_amd import build
        build.build()
    return m


def _declared():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol(M):
    names = _declared()
    assert len(names) == 15, names
    L = M.lib()
    for n in names:
        assert hasattr(L, n), n
    assert sorted(M.EXPORTS) == names
    # nm view of the dynamic symbol table agrees
    out = os.popen(f"nm -D --defined-only {M.LIB_PATH}").read()
    for n in names:
        assert re.search(rf"\bT {n}\b", out), n


def _cfg(M, **kw):
    base = dict(T=64, d=256, E=8, k=2, f=256, act="bf16", weight="bf16")
    base.update(kw)
    return M.make_config(**base)


FAKE = 0x10000  # a 16-byte aligned address that is never dereferenced


def _route(M, c, x=FAKE, ws=None):
    L = M.lib()
    return L.moe_route(ctypes.byref(c), x, FAKE, None, FAKE, FAKE, FAKE, None, ws, 0, None)


def test_config_validation(M):
    L = M.lib()
    bad = [dict(k=9), dict(k=0), dict(d=200), dict(f=100), dict(E=0), dict(E=2000),
           dict(T=-1), dict(k=17, E=32), dict(num_groups=3), dict(num_groups=4, topk_groups=5),
           dict(num_groups=4, topk_groups=2, score="softmax"),
           dict(E=16, k=5, num_groups=4, topk_groups=1, score="sigmoid")]
    for kw in bad:
        assert _route(M, _cfg(M, **kw)) == -1, kw
    assert _route(M, _cfg(M, act="f32", weight="bf16")) == -2
    assert _route(M, _cfg(M, act="f32", weight="fp8")) == -2
    assert _route(M, _cfg(M, weight="fp8", quant_block=64)) == -1
    for tile in (-1, 3):  # MOE_TILE_* is 0, 1 or 2
        c = _cfg(M)
        c.gemm_tile = tile
        assert _route(M, c) == -1, tile
    for coeff in (-0.01, float("nan"), float("inf")):
        assert _route(M, _cfg(M, aux_coeff=coeff)) == -1, coeff
    assert L.moe_workspace_size(ctypes.byref(_cfg(M, k=9)), 1) == 0


def test_size_limits(M):
    """Shapes whose GEMM operands or grids the kernels cannot address are
    refused before any launch: one expert's W1 of 4 GiB or more (32-bit
    buffer offsets from a per-step base), more than 2^38 elements in an
    [A, max(d, 2f)] tensor, more than 2^30 GEMM tiles; and d or f that are
    not multiples of 128, with bf16 and fp32 as with FP8 (the GEMM tiles)."""
    # (valid shapes are seen through moe_workspace_size, which launches
    # nothing: it returns 0 for a refused configuration)
    ws = lambda **kw: M.lib().moe_workspace_size(ctypes.byref(_cfg(M, **kw)), 3)
    # W1 = [2f, d]: 2 * 2^15 * 2^15 * 2 bytes = 4 GiB in bf16 (refused),
    # 2 GiB in fp8 (taken), 4 GiB in fp32 at f = 2^14 (refused)
    assert _route(M, _cfg(M, d=1 << 15, f=1 << 15)) == -1 and ws(d=1 << 15, f=1 << 15) == 0
    assert ws(d=1 << 15, f=1 << 15, weight="fp8") > 0
    assert ws(d=1 << 15, f=(1 << 15) - 128) > 0
    assert _route(M, _cfg(M, d=1 << 15, f=1 << 14, act="f32", weight="f32")) == -1
    assert ws(d=1 << 15, f=(1 << 14) - 128, act="f32", weight="f32") > 0
    # A * max(d, 2f) > 2^38 elements: T = 2^26 tokens, k = 16, d = 2^13
    assert _route(M, _cfg(M, T=1 << 26, E=16, k=16, d=1 << 13, f=128)) == -1
    assert ws(T=1 << 26, E=16, k=16, d=256, f=128) > 0    # exactly 2^38
    # (the tile-count limits follow from these two: under 4 GiB per W1 and
    # 2^38 elements, no GEMM has more than 2^28 tiles)
    for d, f, act in ((1000, 256, "bf16"), (256, 1000, "bf16"), (136, 256, "f32"), (256, 264, "f32")):
        assert _route(M, _cfg(M, d=d, f=f, act=act, weight=act)) == -1, (d, f, act)


def test_dispatch_scratch_refusals(M):
    """The allocation-free dispatch refuses, before any device call, a
    configuration whose workspace exceeds its device array, and the argument
    errors of moe_dispatch."""
    L = M.lib()
    N = None
    big = _cfg(M, T=1 << 21, E=1024, d=128)        # 8192 chunks x 1024 experts x 4 B = 32 MiB
    assert L.moe_workspace_size(ctypes.byref(big), 1) > (8 << 20)
    assert L.moe_dispatch_scratch(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, N, N) == -4
    assert L.moe_dispatch_scratch(ctypes.byref(_cfg(M, k=9)), *([FAKE] * 7), N, N) == -1
    assert L.moe_dispatch_scratch(ctypes.byref(_cfg(M, T=0)), N, N, N, FAKE, N, N, N, N, N) == -1


def test_route_dispatch_refusals(M):
    """The fused route and dispatch checks the arguments of both calls before
    it enqueues either: a bad dispatch argument leaves the routing outputs
    untouched too."""
    L = M.lib()
    N = None
    c = _cfg(M)
    need = L.moe_workspace_size(ctypes.byref(c), 1)

    def rd(cfg, x=FAKE, w=FAKE, x_scale=None, ws=FAKE, nbytes=need, counts=FAKE):
        return L.moe_route_dispatch(ctypes.byref(cfg), x, w, N, FAKE, FAKE, FAKE, N, counts, FAKE,
                                    FAKE, FAKE, FAKE, x_scale, ws, nbytes, N)
    assert rd(c, ws=None, nbytes=0) == -4          # dispatch workspace missing
    assert rd(c, nbytes=need - 1) == -4            # ... or short
    assert rd(c, w=None) == -1                     # route argument
    assert rd(c, x=FAKE + 4) == -3                 # alignment
    assert rd(_cfg(M, weight="fp8")) == -1         # fp8 needs the scale output
    assert rd(_cfg(M, k=9)) == -1                  # configuration
    assert rd(_cfg(M, T=0), x=None, w=None, ws=None, nbytes=0, counts=None) == -1  # zeros to write


def test_empty_batch_enqueues_nothing(M):
    """T = 0: the calls whose outputs all have T rows return at once and
    accept NULL buffers (an empty tensor has no storage). The calls that
    must still write exact zeros (counts and offsets, expert and router
    weight gradients, the auxiliary loss) require those outputs; this CPU
    test only checks the refusals, which come before any launch."""
    c = _cfg(M, T=0)
    L = M.lib()
    N = None
    assert _route(M, c, x=None) == 0
    assert L.moe_combine(ctypes.byref(c), N, N, N, N, N, N) == 0
    assert L.moe_combine_bwd(ctypes.byref(c), N, N, N, N, N, N, N) == 0
    assert L.moe_dispatch_bwd(ctypes.byref(c), N, N, N, N, N) == 0
    assert L.moe_grouped_ffn(ctypes.byref(c), *([N] * 12), 0, N) == 0
    # zeros to write: the output may not be NULL
    assert L.moe_dispatch(ctypes.byref(c), N, N, N, FAKE, N, N, N, N, N, 0, N) == -1    # counts
    assert L.moe_dispatch(ctypes.byref(c), N, N, FAKE, N, N, N, N, N, N, 0, N) == -1    # offsets
    assert L.moe_grouped_ffn_bwd(ctypes.byref(c), *([N] * 12), N, FAKE, N, 0, N) == -1  # dw1
    assert L.moe_grouped_ffn_bwd(ctypes.byref(c), *([N] * 12), FAKE, N, N, 0, N) == -1  # dw2
    assert L.moe_route_bwd(ctypes.byref(c), *([N] * 9), N, 0, N) == -1                  # dw_router
    ca = _cfg(M, T=0, aux_coeff=0.01)
    assert L.moe_route_aux_loss(ctypes.byref(ca), N, N, N, N, 0, N) == -1


def test_null_alignment_and_workspace_errors(M):
    L = M.lib()
    c = _cfg(M)
    assert _route(M, c, x=None) == -1
    assert _route(M, c, x=FAKE + 4) == -3
    # dispatch with a missing / short workspace
    assert L.moe_dispatch(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0,
                          None) == -4
    need = L.moe_workspace_size(ctypes.byref(c), 1)
    assert need > 0
    assert L.moe_dispatch(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                          need - 1, None) == -4
    # fp8 dispatch needs the scale output
    c8 = _cfg(M, weight="fp8")
    assert L.moe_dispatch(ctypes.byref(c8), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                          need, None) == -1
    # route backward workspace
    assert L.moe_route_bwd(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE,
                           None, 0, None) == -4
    # auxiliary loss: needs a nonzero coefficient, an output and a workspace
    assert L.moe_route_aux_loss(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == -1
    ca = _cfg(M, aux_coeff=0.01)
    assert L.moe_route_aux_loss(ctypes.byref(ca), FAKE, FAKE, None, FAKE, 1 << 20, None) == -1
    assert L.moe_route_aux_loss(ctypes.byref(ca), FAKE, FAKE, FAKE, None, 0, None) == -4
    need = L.moe_workspace_size(ctypes.byref(ca), 5)
    assert L.moe_route_aux_loss(ctypes.byref(ca), FAKE, FAKE, FAKE, FAKE, need - 1, None) == -4
    assert L.moe_route_aux_loss(ctypes.byref(ca), FAKE + 4, FAKE, FAKE, FAKE, need, None) == -3
    # quantiser arguments
    assert L.moe_quantize_fp8_blockwise(FAKE, 7, 4, 4, 1, 1, FAKE, FAKE, None) == -2
    assert L.moe_quantize_fp8_blockwise(FAKE, 1, 4, 4, 0, 1, FAKE, FAKE, None) == -1


def test_workspace_sizes_follow_the_config(M):
    L = M.lib()
    c = _cfg(M, T=1000, E=16, k=4, f=384, d=512)
    ws = lambda op: L.moe_workspace_size(ctypes.byref(c), op)
    assert ws(0) == 0 and ws(2) == 0
    assert ws(1) >= ((1000 + 255) // 256) * 16 * 4
    assert ws(3) >= 1000 * 4 * 2 * 384 * 2
    assert ws(4) >= 1000 * 16 * 4
    assert all(ws(op) % 256 == 0 for op in range(6))
    # the auxiliary loss: two [chunks, E] partial arrays; the router backward
    # grows by the counts and f [E] only when the loss is on
    ca = _cfg(M, T=1000, E=16, k=4, f=384, d=512, aux_coeff=0.01)
    wa = lambda op: L.moe_workspace_size(ctypes.byref(ca), op)
    assert wa(5) >= 2 * 16 * 4 and wa(5) == ws(5)
    assert wa(4) >= ws(4) + 16 * 4 + 16 * 4
    # 1 << 22 tokens: at most 256 chunks of partials
    cb = _cfg(M, T=1 << 22, E=1024, k=2, aux_coeff=0.01)
    assert L.moe_workspace_size(ctypes.byref(cb), 5) == 2 * 256 * 1024 * 4


def test_status_strings(M):
    assert M.moe_status_string(0) == "ok"
    assert "workspace" in M.moe_status_string(-4)
    assert M.moe_status_string(-99) == "unknown status"


def test_recompute_modes(M):
    """MOE_RECOMPUTE_*: 0, 1, 2 only; which saved activations may be NULL;
    the workspace grows by what is no longer saved."""
    L = M.lib()
    for bad in (-1, 3):
        c = _cfg(M)
        c.recompute = bad
        assert _route(M, c) == -1, bad
    A, d, f = 1000 * 4, 512, 384
    sizes = {}
    for mode, rc in M.RECOMPUTE.items():
        c = _cfg(M, T=1000, E=16, k=4, f=f, d=d, recompute=mode)
        sizes[mode] = (L.moe_workspace_size(ctypes.byref(c), 2), L.moe_workspace_size(ctypes.byref(c), 3))
    # forward: H moves to the workspace; backward: + H, and + GU for "full"
    assert sizes["none"][0] == 0
    assert sizes["act"][0] >= A * f * 2 and sizes["full"][0] == sizes["act"][0]
    assert sizes["act"][1] >= sizes["none"][1] + A * f * 2
    assert sizes["full"][1] >= sizes["act"][1] + A * 2 * f * 2
    c8 = _cfg(M, T=1000, E=16, k=4, f=f, d=d, weight="fp8", recompute="act")
    c8n = _cfg(M, T=1000, E=16, k=4, f=f, d=d, weight="fp8")
    assert (L.moe_workspace_size(ctypes.byref(c8), 3)
            >= L.moe_workspace_size(ctypes.byref(c8n), 3) + A * f * 3 + A * (f // 128) * 4)

    def ffn(c, gu, h, hs, ws, n):
        return L.moe_grouped_ffn(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, gu, h, hs,
                                 FAKE, ws, n, None)

    def ffn_bwd(c, gu, h, hs, ws, n):
        return L.moe_grouped_ffn_bwd(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, gu, h,
                                     hs, FAKE, FAKE, FAKE, FAKE, ws, n, None)

    # FP8: both calls need a workspace, so with none given every case below
    # returns an error (NULL: -1, else the missing workspace: -4) before any
    # launch or device access
    for mode, need_gu, need_h in (("none", True, True), ("act", True, False), ("full", False, False)):
        c = _cfg(M, T=64, weight="fp8", recompute=mode)
        for call in (ffn, ffn_bwd):
            assert call(c, FAKE, FAKE, FAKE, None, 0) == -4, (mode, call)
            assert call(c, None, FAKE, FAKE, None, 0) == (-1 if need_gu else -4), (mode, call)
            assert call(c, FAKE, None, FAKE, None, 0) == (-1 if need_h else -4), (mode, call)
            assert call(c, FAKE, FAKE, None, None, 0) == (-1 if need_h else -4), (mode, call)
        # with tokens, a recompute workspace is required
        c1 = _cfg(M, T=64, recompute=mode)
        if mode != "none":
            assert ffn(c1, FAKE, None, None, None, 0) == -4
            assert ffn_bwd(c1, FAKE, None, None, None, 0) == -4


def test_mxfp8_config_and_quantiser_arguments(M):
    L = M.lib()
    c = _cfg(M, weight="mxfp8", quant_block=32, T=0)
    assert _route(M, c) == 0
    assert _route(M, _cfg(M, weight="mxfp8", quant_block=128)) == -1
    assert _route(M, _cfg(M, act="f32", weight="mxfp8", quant_block=32)) == -2
    # the backward holds the column-quantised weights only: no GEMM1 rerun
    assert _route(M, _cfg(M, weight="mxfp8", quant_block=32, recompute="full")) == -2
    assert _route(M, _cfg(M, weight="mxfp8", quant_block=32, recompute="act", T=0)) == 0
    # E8M0 scales take as many bytes as the fp32 1 x 128 scales, and both
    # 8-bit layers keep their weight-gradient operands in token blocks (codes
    # [A, C] and [NB, C] scales: FP8 fp32 per 128-row block, MXFP8 one word of
    # four 32-row E8M0 bytes per 128-row block; NB = (A + 127 E) / 128): the
    # same workspace for every call
    A, E, d, f = 4000, 16, 512, 384
    cm = _cfg(M, T=1000, E=E, k=4, f=f, d=d, weight="mxfp8", quant_block=32)
    cf = _cfg(M, T=1000, E=E, k=4, f=f, d=d, weight="fp8")
    for op in (1, 2, 3):
        assert L.moe_workspace_size(ctypes.byref(cm), op) == L.moe_workspace_size(ctypes.byref(cf), op)
    nb = (A + 127 * E) // 128
    tok = A * (2 * d + 3 * f) + 4 * nb * (2 * d + 3 * f)
    assert L.moe_workspace_size(ctypes.byref(cm), 3) >= tok
    q = L.moe_quantize_mxfp8
    assert q(FAKE, 7, 32, 32, 0, FAKE, FAKE, None) == -2          # dtype
    assert q(FAKE, 1, 32, 48, 0, FAKE, FAKE, None) == -1          # cols % 32 (rows mode)
    assert q(FAKE, 1, 48, 32, 1, FAKE, FAKE, None) == -1          # rows % 32 (column mode)
    assert q(FAKE, 1, 32, 32, 2, FAKE, FAKE, None) == -1          # colwise flag
    assert q(None, 1, 32, 32, 0, FAKE, FAKE, None) == -1          # NULL
    assert q(FAKE + 4, 1, 32, 32, 0, FAKE, FAKE, None) == -3      # alignment (rows mode)
    assert q(FAKE, 1, 0, 32, 0, None, None, None) == 0            # empty: nothing to do
