"""Seeded synthetic workloads for the MoE token path.

This module holds the five named layer shapes and the seeded generators of
their inputs. It contains none of the layer's arithmetic: it only draws
normal samples, scales them by a standard deviation, and casts them to the
stored dtype. Both the CPU oracle (under ``oracle/``) and the GPU library's
tests and benchmark draw their inputs from here, so the two sides always see
the same bits.

Shapes follow the pages' workloads:
  * Mixtral-style, 8 experts, top-2, hidden 4096 (Megatron-Core skill page,
    "Workflow 2: MoE" flags ``--num-experts 8 --moe-router-topk 2
    --hidden-size 4096 --seq-length 4096``).
  * DeepSeek-V3-style, 256 experts, top-8 (Megatron Core MoE summary,
    section 4 "Results"; Hybrid-EP article, Grace Blackwell results).
  * Weight std 0.006 (skill page, "problems" section, ``--init-method-std``).
The pages print no dataset; seeded normal inputs stand in for real token
activations and trained weights.

Seeding: every tensor is drawn with its own CPU ``torch.Generator`` seeded
with ``(seed_base << 16) | (tensor_id << 11) | expert_id``, as fp32
``normal_()``, multiplied by ``std`` in fp32, then cast round-to-nearest-even
to the stored dtype. The CPU generator (a Mersenne twister) keeps only the
low 32 bits of its seed, so the three fields are packed into 32 bits.
Expert weights are drawn per expert so that one expert can be regenerated
alone.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import torch

# tensor ids used in the seed
T_X, T_WR, T_W1, T_W2, T_DY, T_SW1, T_SW2 = 1, 2, 3, 4, 5, 6, 7


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    seed_base: int
    T: int                 # tokens
    d: int                 # hidden size
    E: int                 # routed experts
    k: int                 # top-k
    f: int                 # expert ffn hidden size
    shared: int = 0        # number of shared experts (0 or 1)
    score: str = "softmax"  # "softmax" | "sigmoid"
    renorm: bool = True
    gate_scale: float = 1.0
    num_groups: int = 1
    topk_groups: int = 1
    group_score: str = "top2_sum"  # "top2_sum" | "max"
    act: str = "bf16"      # "f32" | "bf16": dtype of x, y, activations
    weight: str = "bf16"   # "f32" | "bf16" | "fp8" | "mxfp8"
    std: float = 0.02      # std of router and expert weights
    bias: str = "none"     # "none" | "zipf": per-expert router logit bias
    quant_block: int = 128
    aux_coeff: float = 0.0  # load-balancing auxiliary loss coefficient (0: off)

    @property
    def A(self) -> int:
        return self.T * self.k

    def replace(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)

    def describe(self) -> dict:
        return dataclasses.asdict(self)


# The five workloads. Index 0 is the tiny fp32 case, index 1 the
# Mixtral-style layer the throughput figure is quoted on.
CONFIGS = [
    LayerConfig("tiny_fp32", 1, T=256, d=128, E=8, k=2, f=256,
                act="f32", weight="f32", std=0.02),
    LayerConfig("mixtral_bf16", 2, T=4096, d=4096, E=8, k=2, f=14336,
                std=0.02),
    LayerConfig("deepseek_v3_bf16", 3, T=4096, d=7168, E=256, k=8, f=2048,
                shared=1, score="sigmoid", renorm=True, gate_scale=2.5,
                num_groups=8, topk_groups=4, std=0.006),
    LayerConfig("qwen3_skew_bf16", 4, T=16384, d=2048, E=128, k=8, f=768,
                score="softmax", renorm=False, bias="zipf", std=0.02),
    LayerConfig("deepseek_v3_fp8", 5, T=8192, d=7168, E=256, k=8, f=2048,
                shared=1, score="sigmoid", renorm=True, gate_scale=2.5,
                num_groups=8, topk_groups=4, weight="fp8", std=0.006),
]
# The MXFP8 variant of the FP8 workload: 1 x 32 blocks with power-of-two
# (E8M0) scales instead of 1 x 128 / 128 x 128 blocks with fp32 scales
# (Hybrid-EP article, results in MXFP8).
EXTRA_CONFIGS = [
    LayerConfig("deepseek_v3_mxfp8", 6, T=8192, d=7168, E=256, k=8, f=2048,
                shared=1, score="sigmoid", renorm=True, gate_scale=2.5,
                num_groups=8, topk_groups=4, weight="mxfp8", quant_block=32, std=0.006),
]
BY_NAME = {c.name: c for c in CONFIGS + EXTRA_CONFIGS}


def mini(cfg: LayerConfig, T: int, d: int, f: int, E: Optional[int] = None,
         seed_base: Optional[int] = None) -> LayerConfig:
    """A smaller layer with the same routing rule and dtypes as ``cfg``."""
    kw = dict(T=T, d=d, f=f, seed_base=(seed_base if seed_base is not None
                                        else cfg.seed_base + 16))
    if E is not None:
        kw["E"] = E
    return cfg.replace(**kw)


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def master_dtype(cfg: LayerConfig) -> torch.dtype:
    """dtype in which expert weights are drawn (fp8 weights have bf16 masters)."""
    return torch.float32 if cfg.weight == "f32" else torch.bfloat16


def draw(seed_base: int, tensor_id: int, expert_id: int, shape, std: float,
         dtype: torch.dtype, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    if not (0 <= seed_base < 1 << 16 and 0 <= tensor_id < 1 << 5 and 0 <= expert_id < 1 << 11):
        raise ValueError(f"seed fields out of range: {seed_base}, {tensor_id}, {expert_id}")
    g = torch.Generator("cpu")
    g.manual_seed((seed_base << 16) | (tensor_id << 11) | expert_id)
    t = torch.empty(shape, dtype=torch.float32)
    t.normal_(generator=g)
    if std != 1.0:
        t.mul_(std)
    t = t.to(dtype)
    if out is not None:
        out.copy_(t)
        return out
    return t


def x(cfg: LayerConfig) -> torch.Tensor:
    return draw(cfg.seed_base, T_X, 0, (cfg.T, cfg.d), 1.0, torch_dtype(cfg.act))


def dy(cfg: LayerConfig) -> torch.Tensor:
    return draw(cfg.seed_base, T_DY, 0, (cfg.T, cfg.d), 1.0, torch_dtype(cfg.act))


def w_router(cfg: LayerConfig) -> torch.Tensor:
    return draw(cfg.seed_base, T_WR, 0, (cfg.E, cfg.d), cfg.std, torch.float32)


def router_bias(cfg: LayerConfig) -> Optional[torch.Tensor]:
    """Per-expert logit offset that skews the load (a synthetic input).

    ``zipf``: b_e = 1.5 * log(1 / rank_e) with rank_e = e + 1, so expert 0 is
    the hottest. Computed in float64, stored as float32.
    """
    if cfg.bias == "none":
        return None
    if cfg.bias == "zipf":
        b = [1.5 * math.log(1.0 / (e + 1)) for e in range(cfg.E)]
        return torch.tensor(b, dtype=torch.float64).to(torch.float32)
    raise ValueError(cfg.bias)


def expert_w1(cfg: LayerConfig, e: int) -> torch.Tensor:
    """W1 of expert e, [2f, d]: rows 0..f-1 are the gate half, f..2f-1 the up half."""
    return draw(cfg.seed_base, T_W1, e, (2 * cfg.f, cfg.d), cfg.std, master_dtype(cfg))


def expert_w2(cfg: LayerConfig, e: int) -> torch.Tensor:
    """W2 of expert e, [d, f]."""
    return draw(cfg.seed_base, T_W2, e, (cfg.d, cfg.f), cfg.std, master_dtype(cfg))


def shared_w1(cfg: LayerConfig) -> torch.Tensor:
    return draw(cfg.seed_base, T_SW1, 0, (2 * cfg.f, cfg.d), cfg.std, master_dtype(cfg))


def shared_w2(cfg: LayerConfig) -> torch.Tensor:
    return draw(cfg.seed_base, T_SW2, 0, (cfg.d, cfg.f), cfg.std, master_dtype(cfg))


def all_expert_weights(cfg: LayerConfig, device="cpu", threads: int = 8):
    """W1 [E, 2f, d] and W2 [E, d, f] (master dtype), filled expert by expert."""
    dt = master_dtype(cfg)
    w1 = torch.empty((cfg.E, 2 * cfg.f, cfg.d), dtype=dt, device=device)
    w2 = torch.empty((cfg.E, cfg.d, cfg.f), dtype=dt, device=device)

    def one(e):
        w1[e].copy_(expert_w1(cfg, e))
        w2[e].copy_(expert_w2(cfg, e))

    if threads <= 1:
        for e in range(cfg.E):
            one(e)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(one, range(cfg.E)))
    return w1, w2
