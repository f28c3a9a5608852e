"""Seeded synthetic inputs (KV pages and decode queries).

This module only draws random numbers; it holds none of the codec's or the
attention's arithmetic.  Both the GPU path and the CPU oracle consume the exact
bytes it produces.

KV recipe (Laplacian-with-outlier-channels, the value model the technical
review "Lynx: Progressive Speculative KV Cache Transfer for Disaggregated LLM
Inference" describes in Prerequisites §4: centred KV is Laplacian-like and a
few channels hold values ~100x larger):

    X[t, h, d] = (Laplace(0, b=0.5) + off[h, d]) * (100 if d in O_h else 1)

with off ~ Normal(0, std 0.2) per channel and O_h a set of 4 distinct head
dims drawn per kv head; the result is rounded to BF16 (nearest even).
Queries are Normal(0, 1) rounded to BF16.

Two generators implement that recipe:
  * `make_kv_np`    — numpy, bit-reproducible on any host; used for sizes the
                      oracle handles (tests, smoke).
  * `make_kv_torch` — torch on a chosen device (the GPU for multi-GB requests);
                      tests copy what they need back to the host.
"""
from __future__ import annotations

import numpy as np

LAPLACE_B = 0.5
OFFSET_STD = 0.2
OUTLIER_SCALE = 100.0
OUTLIERS_PER_HEAD = 4


def _f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """float32 -> BF16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def make_kv_np(tokens: int, kv_heads: int, head_dim: int, seed: int = 0, layer: int = 0,
               kv_idx: int = 0) -> np.ndarray:
    """[tokens, kv_heads, head_dim] BF16 bit patterns (uint16), seeded by (seed, layer, kv_idx)."""
    rng = np.random.default_rng((seed, layer, kv_idx))
    off = rng.normal(0.0, OFFSET_STD, size=(kv_heads, head_dim))
    scale = np.ones((kv_heads, head_dim))
    for h in range(kv_heads):
        dims = rng.choice(head_dim, size=min(OUTLIERS_PER_HEAD, head_dim), replace=False)
        scale[h, dims] = OUTLIER_SCALE
    lap = rng.laplace(0.0, LAPLACE_B, size=(tokens, kv_heads, head_dim))
    x = ((lap + off[None]) * scale[None]).astype(np.float32)
    return _f32_to_bf16_bits(x)


def make_q_np(batch: int, q_heads: int, head_dim: int, seed: int = 0) -> np.ndarray:
    """[batch, q_heads, head_dim] BF16 bit patterns of Normal(0, 1) queries."""
    rng = np.random.default_rng((seed, 0x51))
    return _f32_to_bf16_bits(rng.standard_normal((batch, q_heads, head_dim)).astype(np.float32))


def make_kv_torch(tokens: int, kv_heads: int, head_dim: int, seed: int = 0, layer: int = 0,
                  kv_idx: int = 0, device="cuda", out=None):
    """Same recipe drawn with torch's generator on `device`; returns a bfloat16 tensor
    [tokens, kv_heads, head_dim] (written into `out` when given)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(((seed * 1_000_003 + layer) * 1_000_003 + kv_idx) & 0x7FFF_FFFF_FFFF_FFFF)
    off = torch.randn((kv_heads, head_dim), generator=g, device=device) * OFFSET_STD
    scale = torch.ones((kv_heads, head_dim), device=device)
    for h in range(kv_heads):
        dims = torch.randperm(head_dim, generator=g, device=device)[:OUTLIERS_PER_HEAD]
        scale[h, dims] = OUTLIER_SCALE
    if out is None:
        out = torch.empty((tokens, kv_heads, head_dim), dtype=torch.bfloat16, device=device)
    step = max(1, (1 << 24) // max(1, kv_heads * head_dim))
    for t0 in range(0, tokens, step):
        t1 = min(tokens, t0 + step)
        u = torch.rand((t1 - t0, kv_heads, head_dim), generator=g, device=device) - 0.5
        # inverse-CDF Laplace draw; |u| < 0.5 strictly except at u = -0.5 (log1p(-1) = -inf), clamp it
        lap = -LAPLACE_B * torch.sign(u) * torch.log1p(-2.0 * u.abs()).clamp_min(-80.0)
        out[t0:t1] = ((lap + off) * scale).to(torch.bfloat16)
    return out


def make_q_torch(batch: int, q_heads: int, head_dim: int, seed: int = 0, device="cuda"):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + 0x51) & 0x7FFF_FFFF_FFFF_FFFF)
    return torch.randn((batch, q_heads, head_dim), generator=g, device=device).to(torch.bfloat16)
