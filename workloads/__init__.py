"""Seeded synthetic inputs for the MoE expert-parallel layout / dispatch / combine path.

This module only draws inputs: routing tables, routing weights, token activations, expert outputs and the
shared-expert bias.  It holds none of the path's arithmetic (no counting, placement, quantisation or
reduction) and is shared by the oracle-side tests and the GPU-side tests and bench alike.

All draws use torch's CPU generator seeded per call, so the same (config, seed) gives the same bytes on any
machine with the same torch build.  Values are rounded to BF16 by torch's own cast.

Workloads (shapes and structure of the pages' benchmarks; no dataset or router trace is involved):

  tiny     128 tok, hidden 256, 8 experts, top-2 uniform distinct, alignment 16, zero padding, BF16 dispatch
  decode   128 tok, hidden 7168, 256 experts, top-8 uniform distinct, alignment 128, FP8 dispatch
           (the low-latency decode shape of the DeepEP benchmark tables)
  prefill  4096 tok, hidden 7168, 256 experts in 8 groups, group-limited gating (top-4 groups by group max
           logit, then top-8 experts by logit), alignment 128, zero padding, FP8 dispatch
           (the DeepSeek-V3 pre-training shape of the DeepEP benchmark)
  ep8      4096 tok, hidden 7168, 256 experts over 8 ranks, this rank = 0 owns experts 0..31, top-8 uniform,
           alignment 128, FP8 dispatch with 7 per-destination send windows
  skewed   16384 tok, hidden 7168, 256 experts, top-6 with Zipf(1.1) expert popularity over a seeded
           permutation (Gumbel-top-k sampling without replacement), alignment 128, zero padding, FP8
           dispatch, combine with a shared-expert bias ~ N(0, 0.1^2)   (the DeepEP-Ascend benchmark shape)
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    num_tokens: int
    hidden: int
    num_experts: int
    num_topk: int
    routing: str            # "uniform" | "grouped" | "zipf"
    expert_alignment: int
    zero_padding: bool
    fp8: bool
    num_ranks: int = 1
    rank: int = 0
    bias: bool = False
    num_groups: int = 0     # grouped routing only
    topk_groups: int = 0
    zipf_s: float = 0.0
    bias_std: float = 0.0


CONFIGS = {
    "tiny": Config("tiny", 128, 256, 8, 2, "uniform", 16, True, False),
    "decode": Config("decode", 128, 7168, 256, 8, "uniform", 128, False, True),
    "prefill": Config("prefill", 4096, 7168, 256, 8, "grouped", 128, True, True, num_groups=8, topk_groups=4),
    "ep8": Config("ep8", 4096, 7168, 256, 8, "uniform", 128, False, True, num_ranks=8, rank=0),
    "skewed": Config("skewed", 16384, 7168, 256, 6, "zipf", 128, True, True, bias=True, zipf_s=1.1,
                     bias_std=0.1),
}
ORDER = ["tiny", "decode", "prefill", "ep8", "skewed"]
DEFAULT_SEEDS = {name: i + 1 for i, name in enumerate(ORDER)}


def _gen(seed: int, stream: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed((int(seed) * 1000003 + stream) & 0x7FFFFFFFFFFFFFFF)
    return g


# ---- routing ------------------------------------------------------------------------------------------

def route_uniform_distinct(T: int, E: int, K: int, gen: torch.Generator) -> torch.Tensor:
    """K distinct experts per token, uniform: a partial Fisher-Yates shuffle of 0..E-1 per token."""
    perm = torch.arange(E, dtype=torch.int64).repeat(T, 1)
    rows = torch.arange(T)
    for i in range(K):
        u = torch.rand(T, generator=gen, dtype=torch.float64)
        j = i + torch.clamp((u * (E - i)).long(), max=E - i - 1)
        a = perm[rows, i].clone()
        perm[rows, i] = perm[rows, j]
        perm[rows, j] = a
    return perm[:, :K].contiguous()


def route_grouped(T: int, E: int, K: int, G: int, topg: int, gen: torch.Generator):
    """Group-limited gating on N(0,1) gate logits: score each of G groups by its largest logit, keep the top
    `topg` groups, then take the top K experts by logit among them (descending logit; ties to lower id).
    Returns (topk_idx int64 [T,K], selected logits float64 [T,K])."""
    logits = torch.randn(T, E, generator=gen, dtype=torch.float32).double()
    per = E // G
    gscore = logits.view(T, G, per).max(dim=2).values
    # stable descending order: ties go to the lower group id
    gorder = torch.sort(-gscore, dim=1, stable=True).indices[:, :topg]
    keep = torch.zeros(T, G, dtype=torch.bool)
    keep.scatter_(1, gorder, True)
    masked = logits.masked_fill(~keep.repeat_interleave(per, dim=1), float("-inf"))
    order = torch.sort(-masked, dim=1, stable=True).indices[:, :K]
    return order.contiguous(), torch.gather(logits, 1, order)


def route_zipf(T: int, E: int, K: int, s: float, gen: torch.Generator) -> torch.Tensor:
    """K distinct experts per token with popularity p(pi(i)) ~ (i+1)^-s over a seeded permutation pi;
    sampling without replacement by Gumbel-top-k on log p (descending key order)."""
    pi = torch.randperm(E, generator=gen)
    logp = torch.empty(E, dtype=torch.float64)
    logp[pi] = -s * torch.log(torch.arange(1, E + 1, dtype=torch.float64))
    u = torch.rand(T, E, generator=gen, dtype=torch.float64).clamp_(min=1e-300)
    keys = logp.unsqueeze(0) - torch.log(-torch.log(u))
    return torch.sort(-keys, dim=1, stable=True).indices[:, :K].contiguous()


def softmax_weights(logits: torch.Tensor) -> torch.Tensor:
    """Routing weights: softmax of the selected logits in float64, rounded to float32."""
    return torch.softmax(logits.double(), dim=1).float().contiguous()


# ---- activations --------------------------------------------------------------------------------------

def normal_bf16(shape, gen: torch.Generator, std: float = 1.0) -> torch.Tensor:
    x = torch.randn(*shape, generator=gen, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(torch.bfloat16)


def make_inputs(cfg: Config | str, seed: int | None = None) -> dict:
    """Routing, weights, activations and (if the config has one) bias, as CPU torch tensors.

    Draw order: routing (stream 1), weights (2), x (3), bias (4)."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    if seed is None:
        seed = DEFAULT_SEEDS.get(cfg.name, 0)
    T, E, K, H = cfg.num_tokens, cfg.num_experts, cfg.num_topk, cfg.hidden
    g_route, g_w, g_x, g_b = (_gen(seed, s) for s in (1, 2, 3, 4))
    if cfg.routing == "uniform":
        topk_idx = route_uniform_distinct(T, E, K, g_route)
        weights = softmax_weights(torch.randn(T, K, generator=g_w, dtype=torch.float32))
    elif cfg.routing == "grouped":
        topk_idx, sel = route_grouped(T, E, K, cfg.num_groups, cfg.topk_groups, g_route)
        weights = softmax_weights(sel)
    elif cfg.routing == "zipf":
        topk_idx = route_zipf(T, E, K, cfg.zipf_s, g_route)
        weights = softmax_weights(torch.randn(T, K, generator=g_w, dtype=torch.float32))
    else:
        raise ValueError(cfg.routing)
    x = normal_bf16((T, H), g_x)
    bias = normal_bf16((T, H), g_b, cfg.bias_std) if cfg.bias else None
    return dict(cfg=cfg, seed=seed, topk_idx=topk_idx, topk_weights=weights, x=x, bias=bias)


def random_expert_outputs(rows: int, hidden: int, seed: int, device="cpu") -> torch.Tensor:
    """Random BF16 expert outputs y [rows, hidden] ~ N(0,1), drawn on `device` with a seeded generator."""
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) * 1000003 + 5) & 0x7FFFFFFFFFFFFFFF)
    return torch.randn(rows, hidden, generator=g, dtype=torch.float32, device=device).to(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """BF16 tensor -> numpy uint16 bit patterns (CPU copy)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
