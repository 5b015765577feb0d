"""Workload shapes and seeded synthetic inputs for the MoE layer hot path.

This module only draws random numbers and fixes shapes; it performs none of the
layer's arithmetic (no projection, scoring, selection, dispatch, MLP or
combine).  Both the GPU path and the CPU oracle are fed from it, so it must
stay free of either side's code.

Shapes follow the models the pages name as examples of MoE layers
("Efficient and portable mixture-of-experts communication", Introduction:
Mixtral 8x7B, DeepSeek R1; "Dual Batch Overlap", Running with DBO:
DeepSeek-V2-Lite).  No dataset or trained weight is involved: every tensor is
drawn from a seeded ``torch.Generator`` on the CPU.

Seeding recipe (one generator per tensor, experts drawn in ascending order):
    generator seed = 1000 * seed + tensor_id
    tensor ids: x=0, router=1, gate=2, up=3, down=4,
                shared gate=5, shared up=6, shared down=7
Distributions:
    x ~ N(0, 1); expert weights ~ N(0, std 0.02);
    router ~ N(0, variance 1/d), or U(-1/sqrt(d), 1/sqrt(d)) where stated;
    router bias (Zipf skew) b_e = -s * ln(e + 1), i.e. the log of an
    unnormalised Zipf(s) weight, expert 0 the most popular.
bf16 tensors are drawn in fp32 and rounded to bf16 (round-to-nearest-even).
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass
from typing import Dict, Optional

import torch

TID_X, TID_ROUTER, TID_GATE, TID_UP, TID_DOWN = 0, 1, 2, 3, 4
TID_SH_GATE, TID_SH_UP, TID_SH_DOWN = 5, 6, 7

EXPERT_WEIGHT_STD = 0.02


@dataclass(frozen=True)
class MoEConfig:
    name: str
    num_tokens: int
    hidden: int
    num_experts: int
    top_k: int
    intermediate: int
    expert_begin: int
    expert_end: int
    num_shared: int
    score: str            # "softmax" | "sigmoid"
    renormalize: bool
    dtype: str            # "f32" | "bf16"
    router_init: str      # "normal" (variance 1/d) | "uniform" (+-1/sqrt(d))
    zipf_s: Optional[float] = None   # router bias b_e = -s ln(e+1)
    dual_microbatch: bool = False
    description: str = ""
    packed_weights: bool = False     # bf16 weight stacks in the MOE_WEIGHTS_PACKED layout
    shared_beside_combine: bool = False  # MOE_SHARED_BESIDE_COMBINE placement of shared experts

    @property
    def num_local(self) -> int:
        return self.expert_end - self.expert_begin

    def with_tokens(self, num_tokens: int) -> "MoEConfig":
        return dataclasses.replace(self, num_tokens=num_tokens)

    def replace(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


CONFIGS: Dict[str, MoEConfig] = {
    "tiny_f32": MoEConfig(
        "tiny_f32", 64, 256, 8, 2, 512, 0, 8, 0, "softmax", True, "f32", "normal",
        description="tiny fp32 layer: T=64 d=256 E=8 top-2 I=512"),
    "mixtral_bf16": MoEConfig(
        "mixtral_bf16", 4096, 4096, 8, 2, 14336, 0, 8, 0, "softmax", True, "bf16", "uniform",
        description="Mixtral-8x7B-shaped layer: T=4096 d=4096 E=8 top-2 I=14336"),
    "dsv2lite_decode": MoEConfig(
        "dsv2lite_decode", 128, 2048, 64, 6, 1408, 0, 64, 2, "softmax", False, "bf16", "normal",
        description="DeepSeek-V2-Lite-shaped decode: T=128 d=2048 E=64 top-6 (not renormalised) "
                    "I=1408, 2 shared experts"),
    "dsv3_prefill_ep": MoEConfig(
        "dsv3_prefill_ep", 4096, 7168, 256, 8, 2048, 0, 32, 0, "sigmoid", True, "bf16", "normal",
        zipf_s=1.1,
        description="DeepSeek-V3-shaped prefill, one GPU's expert share: T=4096 d=7168 E=256 "
                    "(experts 0-31 local) top-8 sigmoid+Zipf(1.1) bias I=2048"),
    "dsv3_dual_microbatch": MoEConfig(
        "dsv3_dual_microbatch", 8192, 7168, 256, 8, 2048, 0, 32, 0, "sigmoid", True, "bf16",
        "normal", zipf_s=1.1, dual_microbatch=True,
        description="two 4096-token microbatches of the DeepSeek-V3-shaped expert share, "
                    "split at the midpoint of T padded to a multiple of 256"),
}

CONFIG_ORDER = ["tiny_f32", "mixtral_bf16", "dsv2lite_decode", "dsv3_prefill_ep",
                "dsv3_dual_microbatch"]


def _gen(seed: int, tid: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(1000 * seed + tid)
    return g


def _cast(t: torch.Tensor, cfg: MoEConfig) -> torch.Tensor:
    return t if cfg.dtype == "f32" else t.to(torch.bfloat16)


def make_tokens(cfg: MoEConfig, seed: int = 0) -> torch.Tensor:
    g = _gen(seed, TID_X)
    return _cast(torch.randn(cfg.num_tokens, cfg.hidden, generator=g, dtype=torch.float32), cfg)


def make_router(cfg: MoEConfig, seed: int = 0):
    """Router weight [E, d] in the activation dtype and optional fp32 bias [E]."""
    g = _gen(seed, TID_ROUTER)
    d, E = cfg.hidden, cfg.num_experts
    if cfg.router_init == "uniform":
        a = 1.0 / math.sqrt(d)
        w = torch.rand(E, d, generator=g, dtype=torch.float32) * (2 * a) - a
    else:
        w = torch.randn(E, d, generator=g, dtype=torch.float32) * (1.0 / math.sqrt(d))
    bias = None
    if cfg.zipf_s is not None:
        bias = torch.tensor([-cfg.zipf_s * math.log(e + 1.0) for e in range(E)],
                            dtype=torch.float32)
    return _cast(w, cfg), bias


def _expert_stack(cfg: MoEConfig, n: int, rows: int, cols: int, seed: int, tid: int):
    g = _gen(seed, tid)
    out = torch.empty(n, rows, cols, dtype=cfg.torch_dtype)
    for e in range(n):
        out[e] = _cast(torch.randn(rows, cols, generator=g, dtype=torch.float32)
                       * EXPERT_WEIGHT_STD, cfg)
    return out


def make_experts(cfg: MoEConfig, seed: int = 0):
    """Local routed experts: gate/up [E_loc, I, d], down [E_loc, d, I] ([out, in] layout)."""
    n, d, I = cfg.num_local, cfg.hidden, cfg.intermediate
    return (_expert_stack(cfg, n, I, d, seed, TID_GATE),
            _expert_stack(cfg, n, I, d, seed, TID_UP),
            _expert_stack(cfg, n, d, I, seed, TID_DOWN))


def make_shared(cfg: MoEConfig, seed: int = 0):
    """Shared (always-applied) experts, same layout as the routed ones, or Nones."""
    n, d, I = cfg.num_shared, cfg.hidden, cfg.intermediate
    if n == 0:
        return None, None, None
    return (_expert_stack(cfg, n, I, d, seed, TID_SH_GATE),
            _expert_stack(cfg, n, I, d, seed, TID_SH_UP),
            _expert_stack(cfg, n, d, I, seed, TID_SH_DOWN))


def make_inputs(cfg: MoEConfig, seed: int = 0, with_experts: bool = True) -> dict:
    """All host tensors of one layer call, keyed by the C-ABI argument names."""
    w_router, bias = make_router(cfg, seed)
    inp = {"x": make_tokens(cfg, seed), "w_router": w_router, "bias": bias}
    if with_experts:
        inp["w_gate"], inp["w_up"], inp["w_down"] = make_experts(cfg, seed)
        inp["ws_gate"], inp["ws_up"], inp["ws_down"] = make_shared(cfg, seed)
    return inp


def random_ids(T: int, E: int, K: int, seed: int, invalid_frac: float = 0.0,
               repeat_pool: int = 0) -> torch.Tensor:
    """Distinct-per-token random expert ids [T, K] int32, for dispatch-only cases.

    With ``invalid_frac`` > 0, that fraction of slots is replaced by out-of-range
    ids (negative or >= E), which the dispatch must skip and count.  With
    ``repeat_pool`` > 0 the slots are drawn with replacement from experts
    [0, repeat_pool) instead, so a token may name an expert more than once.
    """
    g = _gen(seed, 100)
    if repeat_pool > 0:
        ids = torch.randint(0, min(repeat_pool, E), (T, K), generator=g, dtype=torch.int32)
    else:
        ids = torch.argsort(torch.rand(T, E, generator=g), dim=1)[:, :K].to(torch.int32)
    if invalid_frac > 0:
        m = torch.rand(T, K, generator=g) < invalid_frac
        bad = torch.where(torch.rand(T, K, generator=g) < 0.5,
                          torch.full((T, K), -1, dtype=torch.int32),
                          torch.full((T, K), E + 3, dtype=torch.int32))
        ids = torch.where(m, bad, ids)
    return ids.contiguous()
