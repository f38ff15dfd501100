"""Pins of the FP8 split-GEMM oracle (oracle/fp8.py).

The decode is pinned to values the OCP E4M3 definition fixes (named codes,
subnormals, the NaN pattern, the largest finite value) and, for all 256 codes,
to torch's own float8_e4m3fn type; the product is pinned by one-hot and
integer-valued cases with an exact answer.  A wrong bias, dropped subnormals,
a lost sign or a transposed operand each fail one of these."""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import fp8 as of


@pytest.mark.parametrize("code, value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6), (0x38, 1.0), (0x40, 2.0),
    (0x3F, 1.875), (0x44, 3.0), (0x7E, 448.0), (0xFE, -448.0), (0xB8, -1.0), (0x81, -(2.0 ** -9)),
])
def test_named_codes(code, value):
    assert of.decode_e4m3(code) == value


def test_signed_zero_and_nan():
    assert of.decode_e4m3(0x80) == 0.0 and math.copysign(1.0, of.decode_e4m3(0x80)) < 0
    assert math.isnan(of.decode_e4m3(0x7F)) and math.isnan(of.decode_e4m3(0xFF))
    assert sum(math.isnan(v) for v in of.E4M3_TABLE) == 2
    assert np.nanmax(np.abs(of.E4M3_TABLE)) == of.E4M3_MAX


def test_all_codes_match_torch_float8():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(of.E4M3_TABLE, ref, equal_nan=True)


def test_order_and_symmetry():
    pos = of.E4M3_TABLE[:0x7F]
    assert np.all(np.diff(pos) > 0) and pos[0] == 0.0
    assert np.array_equal(of.E4M3_TABLE[0x80:0xFF], -pos)


def test_one_hot_selects_scaled_weight_column():
    codes = synth.fp8_all_codes(32, 48, seed=1).numpy()
    scale = np.linspace(0.5, 2.0, 32)
    cols = [0, 17, 47]
    x = np.zeros((3, 48))
    for n, j in enumerate(cols):
        x[n, j] = 1.0
    y = of.gemm_fp8(codes, scale, x)
    assert y.shape == (3, 32)
    for n, j in enumerate(cols):
        assert np.array_equal(y[n], scale * of.E4M3_TABLE[codes[:, j]])


def test_integer_values_exact():
    # Codes of small integers, power-of-two scales and integer x: exact integers.
    ints = {0x38: 1, 0x40: 2, 0x44: 3, 0x48: 4, 0xB8: -1, 0xC0: -2, 0x00: 0}
    keys = np.array(list(ints), dtype=np.uint8)
    rng = np.random.default_rng(2)
    codes = keys[rng.integers(0, len(keys), (16, 40))]
    scale = 2.0 ** rng.integers(-2, 3, 16)
    x = rng.integers(-3, 4, (5, 40)).astype(np.float64)
    y = of.gemm_fp8(codes, scale, x)
    A = np.vectorize(ints.get)(codes)
    exact = [[float(scale[r]) * sum(int(A[r, k]) * int(x[n, k]) for k in range(40)) for r in range(16)]
             for n in range(5)]
    assert y.tolist() == exact


def test_split_is_independent_of_host_rows():
    codes, scale, x = synth.fp8_gemm_inputs(64, 32, 3, seed=4)
    ref = of.gemm_fp8(codes, scale, x)
    for h in range(0, 64 + 1, 16):
        y = of.split_gemm_fp8(codes[:h], codes[h:], scale, x)
        assert np.array_equal(y, ref)


def test_synth_quantization_is_faithful():
    # The generated codes decode to within e4m3's half-ulp (2^-4 relative) of
    # the drawn weights: the inputs are FP8 weights of an N(0, 0.02) layer.
    gen = torch.Generator().manual_seed(5)
    Af = torch.randn((8, 64), generator=gen) * 0.02
    codes, scale, _ = synth.fp8_gemm_inputs(8, 64, 1, seed=5)
    W = of.decode(codes) * scale.double().numpy()[:, None]
    err = np.abs(W - Af.double().numpy())
    assert np.all(err <= np.abs(Af.double().numpy()) * 2.0 ** -4 + scale.double().numpy()[:, None] * 2.0 ** -10)
