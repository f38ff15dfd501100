"""Oracle of the split GEMM over FP8 (e4m3) weights.

Test infrastructure only: nothing on the product path imports this module.

The BOOST page (§5 "Evaluation", Models) runs its models in FP8, and its
offloading page notes that FP8 halves the bytes per layer; neither fixes the
encoding or the scaling.  Read here as: each weight is an OCP FP8 E4M3 code
(the "fn" variant: no infinities, one NaN pattern per sign) and each output row
r of A carries one fp32 scale s[r], so the logical weight is s[r] * e4m3(A[r,k]);
activations stay bf16.  The split is the same as for bf16 weights (DAK §4.1):
the first h tile-rows live in host memory, the result does not depend on h.

    y[n, r] = s[r] * sum_k e4m3(A[r, k]) * x[n, k]

All arithmetic is fp64, exact on the widened inputs.
"""
from __future__ import annotations

import numpy as np

E4M3_BIAS = 7
E4M3_MAX = 448.0


def decode_e4m3(code: int) -> float:
    """Value of one OCP E4M3 code (an int in [0, 255]) from the format's fields:
    sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0.  Exponent 0
    holds the subnormals m / 8 * 2^(1 - 7); the all-ones exponent with mantissa
    7 is NaN (there is no infinity); every other code is (1 + m / 8) * 2^(e - 7)."""
    if not 0 <= code <= 255:
        raise ValueError("an e4m3 code is one byte")
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (1 - E4M3_BIAS)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - E4M3_BIAS)


# All 256 values, index = code (a table of the definition above).
E4M3_TABLE = np.array([decode_e4m3(c) for c in range(256)], dtype=np.float64)


def decode(codes) -> np.ndarray:
    """Decode an array of e4m3 codes (uint8 numpy array or torch tensor) to fp64."""
    if hasattr(codes, "detach"):
        codes = codes.detach().to("cpu").numpy()
    c = np.asarray(codes)
    if c.dtype != np.uint8:
        raise ValueError("codes must be uint8")
    return E4M3_TABLE[c]


def gemm_fp8(codes, scale, x) -> np.ndarray:
    """y [N, M] = s[r] * sum_k e4m3(A[r, k]) x[n, k] in fp64.

    codes: uint8 [M, K]; scale: [M] (fp32 values, widened); x: [N, K] (bf16
    values, widened)."""
    A = decode(codes)
    s = np.asarray(scale.detach().to("cpu").double().numpy() if hasattr(scale, "detach") else scale,
                   dtype=np.float64)
    xs = np.asarray(x.detach().to("cpu").double().numpy() if hasattr(x, "detach") else x, dtype=np.float64)
    if A.ndim != 2 or xs.ndim != 2 or xs.shape[1] != A.shape[1] or s.shape != (A.shape[0],):
        raise ValueError("shapes: codes [M, K], scale [M], x [N, K]")
    return (xs @ A.T) * s[None, :]


def split_gemm_fp8(codes_host, codes_hbm, scale, x) -> np.ndarray:
    """The same product over A = [host rows; HBM rows] (DAK §4.1): each tier's
    rows produce their own output rows."""
    parts = [c for c in (codes_host, codes_hbm) if c is not None and len(c)]
    codes = np.concatenate([np.asarray(c.detach().to("cpu").numpy() if hasattr(c, "detach") else c)
                            for c in parts], axis=0)
    return gemm_fp8(codes, scale, x)
