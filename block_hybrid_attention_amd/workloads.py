"""Seeded synthetic inputs for block-hybrid attention.

This module only draws random numbers and names workload shapes; it holds
none of the method's arithmetic.  Tests hand the same tensors to the HIP
library and to the fp64 oracle, and the benchmark draws its inputs here.

Workload shapes follow the kernel microbenchmark of "Retrofitting Linear
Attention into Diffusion Language Models" (Appendix A: one 32-token block per
request, P tokens of committed context, batches of requests) and the serving
setting of section 4 (128 concurrent requests).  The pages do not give the
model's head count, head_dim or feature width, so H=16, d=128, F=128 are this
library's choice.  q, k, v ~ N(0,1); W ~ N(0, 1/d); bf16 values are fp32
draws rounded to nearest-even by torch.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    block: int
    head_dim: int
    feat: int              # F; the feature map has 2F entries
    dtype: torch.dtype     # q, k, v, W (and the comparator's KV cache)
    seed: int
    prefix: tuple = field(default=())   # per-request committed prefix lengths (tokens)
    note: str = ""


TINY_FP32 = Workload("tiny_fp32", batch=1, heads=1, block=8, head_dim=64, feat=64,
                     dtype=torch.float32, seed=1, prefix=(32,),
                     note="4 committed 8-token blocks, then one step")
BF16_B8 = Workload("bf16_b8_p2048", batch=8, heads=16, block=32, head_dim=128, feat=128,
                   dtype=torch.bfloat16, seed=2, prefix=(2048,) * 8,
                   note="2048-token prefix committed, then one step")
SERVING_B128_SEED = 3
DECODE_B32_SEED = 4_000_000
COMPARATOR_PREFIXES = (1024, 4096, 16384, 32768)


def serving_prefix_lengths(batch: int = 128, seed: int = SERVING_B128_SEED, block: int = 32,
                           lo_blocks: int = 16, hi_blocks: int = 128) -> tuple:
    """Per-request prefix lengths uniform in [512, 4096] tokens, whole blocks."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    nb = torch.randint(lo_blocks, hi_blocks + 1, (batch,), generator=g)
    return tuple(int(x) * block for x in nb)


def serving_b128() -> Workload:
    return Workload("serving_b128", batch=128, heads=16, block=32, head_dim=128, feat=128,
                    dtype=torch.bfloat16, seed=SERVING_B128_SEED,
                    prefix=serving_prefix_lengths(),
                    note="prefix uniform in [512,4096] tokens, rounded to 32-token blocks")


def generator(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=torch.device(device).type if str(device) != "cpu" else "cpu")
    g.manual_seed(int(seed))
    return g


def normal(shape, std: float, dtype: torch.dtype, gen: torch.Generator, device) -> torch.Tensor:
    """std * N(0,1) drawn in fp32 on ``device`` and rounded to ``dtype``."""
    x = torch.randn(tuple(shape), generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def feature_weights(heads: int, head_dim: int, feat: int, dtype, gen, device) -> torch.Tensor:
    """W [H][d][F] ~ N(0, 1/d)."""
    return normal((heads, head_dim, feat), head_dim ** -0.5, dtype, gen, device)


def block_qkv(batch: int, heads: int, tokens: int, head_dim: int, dtype, gen, device):
    """q, k, v [B][H][T][d] ~ N(0,1)."""
    return tuple(normal((batch, heads, tokens, head_dim), 1.0, dtype, gen, device)
                 for _ in range(3))


def gate_from_alpha(heads: int, gen, device) -> torch.Tensor:
    """w = sigma(alpha) with alpha ~ N(0,1): the learned per-head gate's form."""
    a = torch.randn((heads,), generator=gen, device=device, dtype=torch.float32)
    return torch.sigmoid(a)
