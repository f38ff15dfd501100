"""Seeded synthetic inputs for the split operators.

This module is shared by the CPU oracle checks, the GPU parity tests and the
benchmark.  It holds none of the method's arithmetic: it draws random numbers
and rounds them to bf16, nothing else.

Recipe (every generator):
  * a ``torch.Generator`` seeded with ``seed`` (CPU unless ``device`` says otherwise);
  * standard normals drawn as fp32, in the order the function documents;
  * multiplied by the stated standard deviation ("N(0, s)" is read as std = s);
  * rounded to bf16 with round-to-nearest-even (``Tensor.to(torch.bfloat16)``).

Shapes follow Llama-style decode: weights A are [M, K] row-major, activations
are stored as x [N, K] row-major (the K x N operand B of C = A.B held
column-major), K/V caches are [B, Hkv, ctx, D] row-major.
"""
from __future__ import annotations

import torch

__all__ = [
    "normal_bf16",
    "gemm_inputs",
    "int_valued_bf16",
    "attn_inputs",
    "LLAMA8B_LINEARS",
    "LLAMA70B_LINEARS",
]

# (name, M, K) of the Llama-8B decode linears (QKV fused, O, gate+up fused, down)
LLAMA8B_LINEARS = (
    ("qkv", 6144, 4096),
    ("o", 4096, 4096),
    ("gate_up", 28672, 4096),
    ("down", 4096, 14336),
)
# (name, M, K) of the Llama-70B decode linears (hidden 8192, GQA 64/8, hd 128, FFN 28672)
LLAMA70B_LINEARS = (
    ("qkv", 10240, 8192),
    ("o", 8192, 8192),
    ("gate_up", 57344, 8192),
    ("down", 8192, 28672),
)


def normal_bf16(shape, std: float, gen: torch.Generator, device=None) -> torch.Tensor:
    """std * N(0,1) drawn as fp32 from ``gen`` and rounded to bf16."""
    dev = device if device is not None else gen.device
    t = torch.randn(tuple(shape), generator=gen, dtype=torch.float32, device=dev)
    if std != 1.0:
        t.mul_(std)
    return t.to(torch.bfloat16)


def gemm_inputs(M: int, K: int, N: int, seed: int = 0, a_std: float = 0.02,
                x_std: float = 1.0, device=None):
    """Weights A [M, K] ~ N(0, a_std) then activations x [N, K] ~ N(0, x_std), both bf16.

    Draw order: all of A, then all of x.
    """
    gen = torch.Generator(device=device if device is not None else "cpu").manual_seed(seed)
    A = normal_bf16((M, K), a_std, gen)
    X = normal_bf16((N, K), x_std, gen)
    return A, X


def fp8_gemm_inputs(M: int, K: int, N: int, seed: int = 0, a_std: float = 0.02, x_std: float = 1.0,
                    device=None):
    """FP8 weights as a checkpoint would hold them: codes [M, K] uint8 (OCP
    E4M3), one fp32 scale per row [M], and activations x [N, K] bf16.

    Weights are drawn ~N(0, a_std) in fp32, each row is scaled so that its
    largest magnitude maps to 448 (the largest finite e4m3 value) and cast to
    e4m3 by torch's round-to-nearest-even cast; x ~N(0, x_std) in bf16.
    Draw order: all of A, then all of x."""
    gen = torch.Generator(device=device if device is not None else "cpu").manual_seed(seed)
    Af = torch.randn((M, K), generator=gen, device=gen.device, dtype=torch.float32) * a_std
    scale = (Af.abs().amax(dim=1) / 448.0).clamp_min(2.0 ** -100)
    codes = (Af / scale[:, None]).to(torch.float8_e4m3fn).view(torch.uint8)
    X = normal_bf16((N, K), x_std, gen)
    return codes, scale, X


def fp8_all_codes(M: int, K: int, seed: int = 0, device=None) -> torch.Tensor:
    """uint8 [M, K] with every finite e4m3 code (all but 0x7F and 0xFF) drawn
    uniformly: covers zeros, subnormals, both signs and +-448."""
    gen = torch.Generator(device=device if device is not None else "cpu").manual_seed(seed)
    finite = torch.tensor([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=torch.uint8, device=gen.device)
    idx = torch.randint(0, finite.numel(), (M, K), generator=gen, device=gen.device)
    return finite[idx]


def int_valued_bf16(shape, lo: int, hi: int, seed: int = 0) -> torch.Tensor:
    """Integers drawn uniformly from [lo, hi] (inclusive), stored exactly in bf16."""
    gen = torch.Generator().manual_seed(seed)
    t = torch.randint(lo, hi + 1, tuple(shape), generator=gen, dtype=torch.int64)
    return t.to(torch.bfloat16)


def attn_inputs(B: int, Hq: int, Hkv: int, D: int, ctx: int, seed: int = 0,
                std: float = 1.0, device=None):
    """q [B, Hq, D], K [B, Hkv, ctx, D], V [B, Hkv, ctx, D], all bf16 ~ N(0, std).

    Draw order: all of q, then for each request b in index order K[b] then V[b].
    """
    gen = torch.Generator(device=device if device is not None else "cpu").manual_seed(seed)
    dev = gen.device
    q = normal_bf16((B, Hq, D), std, gen)
    K = torch.empty((B, Hkv, ctx, D), dtype=torch.bfloat16, device=dev)
    V = torch.empty((B, Hkv, ctx, D), dtype=torch.bfloat16, device=dev)
    for b in range(B):
        K[b] = normal_bf16((Hkv, ctx, D), std, gen)
        V[b] = normal_bf16((Hkv, ctx, D), std, gen)
    return q, K, V
