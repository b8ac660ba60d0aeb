"""moe_dispatch_scratch (the dispatch for callers that cannot allocate: its
workspace is a device array inside the library) against moe_dispatch with a
caller-owned workspace, through the C ABI: every output bit for bit, on two
calls in a row, the second on a smaller input (the array keeps the first
call's contents), and against the oracle's indices."""
import numpy as np
import pytest
import torch

import moe_synth as S
import oracle

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _outputs(cfg):
    A, fp8 = cfg.A, cfg.weight in ("fp8", "mxfp8")
    o = dict(counts=torch.full((cfg.E,), -7, dtype=torch.int32, device=DEV),
             offsets=torch.full((cfg.E + 1,), -7, dtype=torch.int32, device=DEV),
             rmap=torch.full((cfg.T, cfg.k), -7, dtype=torch.int32, device=DEV),
             ptok=torch.full((A,), -7, dtype=torch.int32, device=DEV))
    if fp8:
        o["xp"] = torch.full((A, cfg.d), 0x55, dtype=torch.uint8, device=DEV)
        o["xs"] = torch.full((A, cfg.d // 128), float("nan"), dtype=torch.float32, device=DEV)
    else:
        o["xp"] = torch.full((A, cfg.d), float("nan"), dtype=torch.bfloat16, device=DEV)
        o["xs"] = None
    return o


def _call(fn, cfg, x, idx, o, ws=None):
    from mixture_experts_layer_gather_amd import make_config
    c = make_config(**cfg.describe())
    args = (c, x, idx, o["counts"], o["offsets"], o["rmap"], o["ptok"], o["xp"], o["xs"])
    fn(*args) if ws is None else fn(*args, ws)
    torch.cuda.synchronize()


CASES = [S.mini(S.BY_NAME["qwen3_skew_bf16"], T=3000, d=256, f=128, E=64).replace(k=4),      # bf16, 12 chunks
         S.mini(S.BY_NAME["deepseek_v3_fp8"], T=700, d=256, f=128, E=32).replace(k=6)]        # fp8, smaller


def test_dispatch_scratch_matches_dispatch():
    from mixture_experts_layer_gather_amd import (make_config, moe_dispatch, moe_dispatch_scratch,
                                                   workspace_size)
    for cfg in CASES:
        print(f"[scratch] {cfg.name} T={cfg.T} E={cfg.E} k={cfg.k} d={cfg.d} {cfg.weight}", flush=True)
        x = S.x(cfg)
        _, idx, _ = oracle.route(cfg, x, S.w_router(cfg), S.router_bias(cfg))
        counts, offsets, rmap, ptok = oracle.dispatch_index(idx, cfg.E)
        xd, idd = x.to(DEV), torch.from_numpy(idx).to(DEV)
        ws = torch.empty(workspace_size(make_config(**cfg.describe()), 1), dtype=torch.uint8, device=DEV)
        ref = _outputs(cfg)
        _call(moe_dispatch, cfg, xd, idd, ref, ws)
        got = _outputs(cfg)
        _call(moe_dispatch_scratch, cfg, xd, idd, got)
        for n in ref:
            if ref[n] is not None:
                assert torch.equal(ref[n].view(torch.uint8), got[n].view(torch.uint8)), n
        assert np.array_equal(got["counts"].cpu().numpy(), counts)
        assert np.array_equal(got["offsets"].cpu().numpy(), offsets)
        assert np.array_equal(got["rmap"].cpu().numpy(), rmap)
        assert np.array_equal(got["ptok"].cpu().numpy(), ptok)


def test_dispatch_scratch_refuses_a_config_past_its_array():
    from mixture_experts_layer_gather_amd import MoeError, moe_dispatch_scratch, make_config
    # ceil(2^21 / 256) chunks x 1024 experts x 4 bytes = 32 MiB > 8 MiB: refused
    # on the host, before any launch (the buffers are never touched)
    c = make_config(T=1 << 21, d=128, E=1024, k=2, f=128)
    t = torch.empty(16, dtype=torch.int32, device=DEV)
    with pytest.raises(MoeError) as e:
        moe_dispatch_scratch(c, t, t, t, t, t, t, t)
    assert e.value.rc == -4
