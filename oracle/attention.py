"""Oracle of the split decode attention (DAK paper §5 "Implementation",
"Supporting FlashAttention"; walkthrough section on the batch split of the KV cache).

The KV cache is partitioned along the batch: requests [0, h) keep their K/V in
host memory, the rest in HBM.  Each request attends only to its own cache, so the
split changes where bytes come from but not the result; attention stays exact.

Per request b and query head j (one query token, no mask, every position valid):
  g    = j // (Hq // Hkv)                      (grouped-query attention: consecutive
                                                query heads share one KV head)
  s_t  = scale * sum_d q[b, j, d] * K[b, g, t, d]
  p_t  = exp(s_t - max_t s_t) / sum_t exp(s_t - max_t s_t)
  o[d] = sum_t p_t * V[b, g, t, d]
All in fp64 on exactly-widened bf16 inputs.
"""
from __future__ import annotations

import numpy as np


def kv_group(j: int, Hq: int, Hkv: int) -> int:
    """KV head read by query head j."""
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return j // (Hq // Hkv)


def attend_one(q_j: np.ndarray, K_g: np.ndarray, V_g: np.ndarray, scale: float) -> np.ndarray:
    """Softmax attention of one query vector q_j [D] over K_g, V_g [T, D]."""
    q_j = np.asarray(q_j, dtype=np.float64)
    K_g = np.asarray(K_g, dtype=np.float64)
    V_g = np.asarray(V_g, dtype=np.float64)
    s = scale * (K_g @ q_j)
    e = np.exp(s - np.max(s))
    p = e / np.sum(e)
    return p @ V_g


def decode_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """out [B, Hq, D] for q [B, Hq, D] and K, V [B, Hkv, T, D]."""
    B, Hq, D = q.shape
    Hkv = K.shape[1]
    out = np.empty((B, Hq, D), dtype=np.float64)
    for b in range(B):
        for j in range(Hq):
            g = kv_group(j, Hq, Hkv)
            out[b, j] = attend_one(q[b, j], K[b, g], V[b, g], scale)
    return out


def decode_attention_lens(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float, lens) -> np.ndarray:
    """``decode_attention`` over a ragged batch: request b attends to its first
    lens[b] positions only (the cache holds T positions per request; those
    past lens[b] are storage, not context)."""
    B, Hq, D = q.shape
    Hkv = K.shape[1]
    out = np.empty((B, Hq, D), dtype=np.float64)
    for b in range(B):
        n = int(lens[b])
        if not 1 <= n <= K.shape[2]:
            raise ValueError("every request needs 1..T valid positions")
        for j in range(Hq):
            g = kv_group(j, Hq, Hkv)
            out[b, j] = attend_one(q[b, j], K[b, g, :n], V[b, g, :n], scale)
    return out


def split_decode_attention(q, K_host, V_host, K_hbm, V_hbm, scale: float) -> np.ndarray:
    """Same as ``decode_attention`` with requests [0, h) taken from the host arrays
    and the remaining requests from the HBM arrays (batch split of the KV cache)."""
    h = K_host.shape[0]
    B = q.shape[0]
    out = np.empty(q.shape, dtype=np.float64)
    if h:
        out[:h] = decode_attention(q[:h], K_host, V_host, scale)
    if B - h:
        out[h:] = decode_attention(q[h:], K_hbm, V_hbm, scale)
    return out
