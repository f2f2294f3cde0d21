"""Seeded synthetic inputs shared by the tests, the bench and smoke().

This module only draws random numbers and describes workload shapes; it holds
none of the method's arithmetic (no pooling, MLP, masking or attention).

Every tensor is drawn as float32 N(0, 1) from a seeded torch generator and,
where the workload is bf16, rounded once to bf16 (round-to-nearest-even, what
torch's conversion does).  The oracle consumes the very bits the GPU sees,
widened to float64, so the generators need no CPU twin.

Workloads (synthetic stand-ins for the long-context evaluations the pages
run on real Qwen3 / Llama-3.1 weights; shapes follow those models):
  tiny      -- 1 x 512 tokens, 2 layers, 4 q / 2 kv heads, d 64, router
               256 -> 64 -> 2, SA blocks of 64 with 1 sink + 2 local blocks.
  prefill32k-- Qwen3-4B-shaped layer: 32768 tokens, 32 q / 8 kv heads, d 128,
               FA and SA on identical inputs, SA blocks of 128, 1 sink block,
               window 2048 tokens (16 blocks incl. the diagonal).
  decode32k -- Qwen3-4B-shaped decode: 16 sequences x 32768 cached tokens,
               36 layers with distinct caches, exactly 18 seeded SA layers.
  prefill128k-- 131072 tokens, 36 layers, router 2560 -> 256 -> 36,
               SA window 4096 tokens (32 blocks).
  varlen8   -- Llama-3-8B-shaped: 8 prompts, lengths uniform in
               [8192, 65536], 32 layers, router 4096 -> 256 -> 32, then 128
               decode steps.
"""

from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    seqlens: tuple           # prompt lengths (prefill) or cache lengths (decode)
    n_layers: int
    hq: int
    hkv: int
    head_dim: int
    block_size: int
    sink_blocks: int
    local_blocks: int        # window in blocks, diagonal block included
    hidden_dim: int = 0      # router input width (0: no router in the workload)
    router_h1: int = 0
    decode_steps: int = 0
    n_sa_layers: int = -1    # decode: exact number of SA layers (-1: router decides)
    extra: dict = field(default_factory=dict)


TINY = Workload("tiny", 1001, (512,), 2, 4, 2, 64, 64, 1, 2, hidden_dim=256, router_h1=64)
PREFILL32K = Workload("prefill32k", 1002, (32768,), 2, 32, 8, 128, 128, 1, 16,
                      hidden_dim=2560, router_h1=256)
DECODE32K = Workload("decode32k", 1003, (32768,) * 16, 36, 32, 8, 128, 128, 1, 16,
                     n_sa_layers=18)
PREFILL128K = Workload("prefill128k", 1004, (131072,), 36, 32, 8, 128, 128, 1, 32,
                       hidden_dim=2560, router_h1=256)
VARLEN8_LENGTH_RANGE = (8192, 65536)


def varlen_lengths(n, lo, hi, seed):
    """n prompt lengths drawn uniformly from the integers in [lo, hi]."""
    g = torch.Generator().manual_seed(seed)
    return tuple(int(x) for x in torch.randint(lo, hi + 1, (n,), generator=g))


def varlen8():
    return Workload("varlen8", 1005, varlen_lengths(8, *VARLEN8_LENGTH_RANGE, 1005),
                    32, 32, 8, 128, 128, 1, 16, hidden_dim=4096, router_h1=256,
                    decode_steps=128)


def generator(seed, device="cpu"):
    return torch.Generator(device=device).manual_seed(int(seed))


def normal(shape, gen, device="cpu", dtype=torch.bfloat16):
    """float32 N(0,1) draws, rounded once to ``dtype``."""
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    return x if dtype == torch.float32 else x.to(dtype)


def router_weights(d_in, h1, n_layers, seed, std=0.02):
    """Router weights N(0, std^2), float32, drawn in the order W1, b1, W2, b2
    from one seeded stream.  PyTorch layout: W1 [h1][d_in], W2 [L][h1]."""
    g = generator(seed)
    w1 = torch.randn((h1, d_in), generator=g) * std
    b1 = torch.randn((h1,), generator=g) * std
    w2 = torch.randn((n_layers, h1), generator=g) * std
    b2 = torch.randn((n_layers,), generator=g) * std
    return w1, b1, w2, b2


def seeded_route(n_layers, n_sa, seed):
    """uint8 route vector with exactly ``n_sa`` SA layers (0) at seeded
    positions, the rest FA (1)."""
    g = generator(seed)
    perm = torch.randperm(n_layers, generator=g)
    route = torch.ones(n_layers, dtype=torch.uint8)
    route[perm[:n_sa]] = 0
    return route


def cu_seqlens(seqlens, device="cpu"):
    c = [0]
    for s in seqlens:
        c.append(c[-1] + int(s))
    return torch.tensor(c, dtype=torch.int32, device=device)
