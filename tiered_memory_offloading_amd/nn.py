"""Drop-in PyTorch modules over the split operators.

DAK paper §5 "Implementation" (PyTorch interface, Supporting FlashAttention):
the kernels are exposed as two modules, SplitK_GEMM for nn.Linear and
SplitK_FlashAttn for scaled dot-product attention, which a model adopts by
swapping its layers at initialisation.  Each module owns its placement: the
first h tile-rows of the weight (or the first h requests of the KV cache) in
pinned host memory, the rest in HBM, with h = ceil(ratio * n) for a given
offload ratio.  The modules only marshal arguments; all arithmetic runs in the
library's kernels (bf16 inputs, fp32 accumulation).
"""
from __future__ import annotations

import math
from fractions import Fraction
from typing import Optional, Union

import torch

from . import (KV_UNIT_HEAD, KV_UNIT_REQUEST, decode_attn_workspace_bytes, place_kv, place_matrix,
               splitk_decode_attn, splitk_gemm)

Ratio = Union[float, Fraction]


def host_units(ratio: Ratio, n: int) -> int:
    """h = ceil(ratio * n) in exact rationals (a float ratio is read as its
    shortest decimal, so 0.1 * 10 gives 1), clamped to [0, n]."""
    r = ratio if isinstance(ratio, Fraction) else Fraction(repr(float(ratio)))
    if r < 0 or r > 1:
        raise ValueError("the offload ratio must lie in [0, 1]")
    return min(n, -((-r.numerator * n) // r.denominator))


class SplitK_GEMM(torch.nn.Module):
    """y = x W^T (+ b) with W's first h tile-rows of m rows in pinned host memory.

    Same call as nn.Linear: input [..., in_features] (bf16), output [...,
    out_features] in `out_dtype` (default: the input's dtype).  The product is
    accumulated in fp32; the bias is added to the fp32 result."""

    def __init__(self, weight: torch.Tensor, bias: Optional[torch.Tensor] = None, host_ratio: Ratio = 0.0,
                 m: int = 64, out_dtype: Optional[torch.dtype] = None):
        super().__init__()
        if weight.dim() != 2:
            raise ValueError("weight must be 2-D [out_features, in_features]")
        self.out_features, self.in_features = weight.shape
        if self.out_features % m:
            raise ValueError(f"out_features {self.out_features} is not a multiple of the tile-row height {m}")
        self.m = m
        self.h = host_units(host_ratio, self.out_features // m)
        w = weight.detach().to(torch.bfloat16)
        self.split = place_matrix(w.cuda() if not w.is_cuda else w, m, self.h)
        self.bias = None if bias is None else bias.detach().to(device="cuda", dtype=torch.float32)
        self.out_dtype = out_dtype

    @classmethod
    def from_linear(cls, linear: torch.nn.Linear, host_ratio: Ratio = 0.0, m: int = 64,
                    out_dtype: Optional[torch.dtype] = None) -> "SplitK_GEMM":
        return cls(linear.weight, linear.bias, host_ratio, m, out_dtype)

    @property
    def host_bytes(self) -> int:
        return self.split.host_bytes

    def forward(self, input: torch.Tensor) -> torch.Tensor:
        if input.shape[-1] != self.in_features:
            raise ValueError(f"input has {input.shape[-1]} features, expected {self.in_features}")
        lead = input.shape[:-1]
        x = input.reshape(-1, self.in_features)
        if x.dtype != torch.bfloat16:
            raise ValueError("input must be bf16 (the split kernels read bf16 activations)")
        x = x.contiguous()
        y = splitk_gemm(self.split, x)
        if self.bias is not None:
            y += self.bias
        y = y.reshape(*lead, self.out_features)
        return y.to(self.out_dtype or input.dtype)


class SplitK_FlashAttn(torch.nn.Module):
    """Decode attention over a KV cache split along the batch: requests
    [0, h) in pinned host memory, the rest in HBM (every request attends within
    one tier).  With unit=KV_UNIT_HEAD the split steps in (request, KV head)
    pairs instead, h = ceil(ratio * B * Hkv); ctx_lens (B integers) gives each
    request's valid cache length for a ragged batch.

    Call as scaled_dot_product_attention for one query token per request:
    query [B, Hq, 1, D] (or [B, Hq, D]) bf16 with Hq a multiple of the cache's
    KV heads (grouped-query attention); no mask, no dropout, not causal (one
    query attends to every cached position).  Output has the query's shape, in
    `out_dtype` (default: the query's dtype)."""

    def __init__(self, key: torch.Tensor, value: torch.Tensor, host_ratio: Ratio = 0.0,
                 out_dtype: Optional[torch.dtype] = None, unit: int = KV_UNIT_REQUEST,
                 ctx_lens: Optional[torch.Tensor] = None):
        super().__init__()
        if key.dim() != 4 or key.shape != value.shape:
            raise ValueError("key and value must be [B, Hkv, ctx, D] of equal shape")
        if unit not in (KV_UNIT_REQUEST, KV_UNIT_HEAD):
            raise ValueError("unit must be KV_UNIT_REQUEST or KV_UNIT_HEAD")
        n = key.shape[0] * (key.shape[1] if unit == KV_UNIT_HEAD else 1)
        self.h = host_units(host_ratio, n)
        self.kv = place_kv(key.detach().to(torch.bfloat16), value.detach().to(torch.bfloat16), self.h,
                           unit=unit, ctx_lens=ctx_lens)
        self.out_dtype = out_dtype
        self._ws = None

    @property
    def host_bytes(self) -> int:
        return self.kv.host_bytes

    def forward(self, query: torch.Tensor, attn_mask=None, dropout_p: float = 0.0, is_causal: bool = False,
                scale: Optional[float] = None) -> torch.Tensor:
        if attn_mask is not None or dropout_p != 0.0 or is_causal:
            raise ValueError("SplitK_FlashAttn takes no mask, no dropout and no causal flag")
        shape = query.shape
        if query.dim() == 4:
            if shape[2] != 1:
                raise ValueError("one query token per request (decode)")
            q = query[:, :, 0, :]
        elif query.dim() == 3:
            q = query
        else:
            raise ValueError("query must be [B, Hq, 1, D] or [B, Hq, D]")
        if q.dtype != torch.bfloat16:
            raise ValueError("query must be bf16")
        B, Hq, D = q.shape
        if B != self.kv.batch or D != self.kv.head_dim:
            raise ValueError("query batch and head_dim must match the KV cache")
        need = decode_attn_workspace_bytes(self.kv, Hq)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty((max(need, 16),), dtype=torch.uint8, device=q.device)
        s = scale if scale is not None else 1.0 / math.sqrt(D)
        out = splitk_decode_attn(q.contiguous(), self.kv, s, ws=self._ws)
        return out.reshape(shape).to(self.out_dtype or query.dtype)
