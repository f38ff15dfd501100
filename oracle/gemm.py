"""Oracle of the split GEMM (DAK paper §4.1 "DAK Design", Fig. 5).

The weight matrix A (M x K) is cut along M into tile-rows of m rows.  The first
h tile-rows live in host memory and the rest in HBM (Fig. 5a puts tile-row 0 on
the host).  Every output row-block depends only on its own tile-row, so the
result C = A.B is the ordinary matrix product of the logical A, whatever h is:
there is no reduction across the split (the "SplitK" name notwithstanding).

Conventions: A is [M, K]; the K x N operand B is held as activations x [N, K];
the product is returned as y [N, M] (y[n, r] = sum_k A[r, k] * x[n, k]).
All arithmetic is fp64 on exactly-widened bf16 inputs.
"""
from __future__ import annotations

from fractions import Fraction
import math

import numpy as np


def to_f64(t) -> np.ndarray:
    """Widen a bf16/fp32 torch tensor or a numpy array to fp64 (exact for bf16)."""
    if hasattr(t, "detach"):
        t = t.detach().to("cpu").float().numpy()
    return np.asarray(t, dtype=np.float64)


def host_units(x, n: int) -> int:
    """Number of units (tile-rows or requests) placed in host memory for ratio x.

    h = ceil(x * n), evaluated in exact rationals so that e.g. x = 0.25 of 16
    tile-rows is exactly 4.  ``x`` may be a Fraction, an int pair (num, den) or a
    float; floats are read as the shortest decimal they print as.
    Rounding up keeps at least the fraction x of the bytes on the host, which is
    what the capacity constraint asks for.
    """
    if isinstance(x, tuple):
        x = Fraction(x[0], x[1])
    elif not isinstance(x, Fraction):
        x = Fraction(repr(float(x)))
    if x < 0 or x > 1:
        raise ValueError("offload ratio must lie in [0, 1]")
    return math.ceil(x * n)


def split_rows(A: np.ndarray, m: int, h: int):
    """Placement of DAK §4.1: (host part = tile-rows [0, h), HBM part = the rest)."""
    M = A.shape[0]
    if M % m:
        raise ValueError("M must be a multiple of the tile-row height m")
    if h < 0 or h * m > M:
        raise ValueError("host tile-row count out of range")
    return A[: h * m], A[h * m:]


def split_gemm(A_host: np.ndarray, A_hbm: np.ndarray, x: np.ndarray) -> np.ndarray:
    """y[n, r] = sum_k A[r, k] x[n, k] for the logical A = [A_host; A_hbm].

    Each tier's rows produce their own output rows; the two results are simply
    placed side by side along M (no cross-tier reduction).
    """
    A_host = np.asarray(A_host, dtype=np.float64)
    A_hbm = np.asarray(A_hbm, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    y_host = x @ A_host.T
    y_hbm = x @ A_hbm.T
    return np.concatenate([y_host, y_hbm], axis=1)


def gemm(A: np.ndarray, x: np.ndarray) -> np.ndarray:
    """The unsplit product y = x . A^T in fp64 (what every split must equal)."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(A, dtype=np.float64).T


def gemm_rows(A_rows: np.ndarray, x: np.ndarray) -> np.ndarray:
    """y[:, rows] for a sample of rows of A (used to check large shapes row by row)."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(A_rows, dtype=np.float64).T


def normwise_error(y, ref) -> float:
    """max |y - ref| / max |ref|: the error measure adopted for outputs near zero."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref)) if ref.size else 0.0
    num = np.max(np.abs(y - ref)) if ref.size else 0.0
    if den == 0.0:
        return 0.0 if num == 0.0 else math.inf
    return float(num / den)
