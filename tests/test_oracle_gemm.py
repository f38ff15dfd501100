"""Pins of the split-GEMM oracle against facts the pages and linear algebra fix.

The oracle (oracle/gemm.py) is C = A.B with A split by tile-rows (DAK paper §4.1).
Each check below would fail on a plausible slip: a transposed operand, rows and
columns swapped, a dropped tier, or a wrong host tile-row count.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import gemm as og


def test_one_hot_columns_select_weight_columns():
    # x[n] = e_{j_n}  =>  y[n, r] = A[r, j_n] exactly (pins orientation: y is [N, M]).
    rng = np.random.default_rng(1)
    M, K = 48, 40
    A = rng.standard_normal((M, K))
    cols = [0, 7, 39]
    x = np.zeros((len(cols), K))
    for n, j in enumerate(cols):
        x[n, j] = 1.0
    y = og.gemm(A, x)
    assert y.shape == (len(cols), M)
    for n, j in enumerate(cols):
        assert np.array_equal(y[n], A[:, j])


def test_rank_one_closed_form():
    # A = u v^T  =>  y[n, r] = u[r] * (v . x[n]).
    u = np.array([1.0, -2.0, 0.5, 4.0])
    v = np.array([2.0, 0.0, -1.0, 3.0, 1.0])
    A = np.outer(u, v)
    x = np.array([[1.0, 2.0, 3.0, 4.0, 5.0], [0.0, -1.0, 0.0, 2.0, 0.5]])
    y = og.gemm(A, x)
    for n in range(2):
        assert np.array_equal(y[n], u * float(v @ x[n]))


def test_integer_inputs_match_exact_integer_product():
    # Integer-valued bf16 inputs: every partial sum is an exact integer, so the
    # fp64 result must equal arbitrary-precision integer arithmetic.
    A = og.to_f64(synth.int_valued_bf16((9, 13), -2, 2, seed=3))
    x = og.to_f64(synth.int_valued_bf16((5, 13), -2, 2, seed=4))
    Ai = A.astype(np.int64).tolist()
    xi = x.astype(np.int64).tolist()
    exact = [[sum(a * b for a, b in zip(Ai[r], xi[n])) for r in range(9)] for n in range(5)]
    assert og.gemm(A, x).tolist() == exact


def test_split_is_independent_of_host_tile_rows():
    # Output rows come from their own tile-row only: any h gives the same y.
    A = og.to_f64(synth.int_valued_bf16((64, 32), -3, 3, seed=5))
    x = og.to_f64(synth.int_valued_bf16((3, 32), -3, 3, seed=6))
    ref = og.gemm(A, x)
    for h in range(0, 64 // 16 + 1):
        Ah, Ag = og.split_rows(A, 16, h)
        assert Ah.shape[0] == 16 * h
        assert np.array_equal(og.split_gemm(Ah, Ag, x), ref)


def test_host_units_config_and_figure_values():
    # x = 0.25 of 16 tile-rows of 64 in a 1024-row matrix: the first 4 tile-rows.
    assert og.host_units(0.25, 1024 // 64) == 4
    # Fig. 4's illustrated splits: 75 % of 16 -> 12, 25 % of 12 -> 3, 33 % of 6 -> 2.
    assert og.host_units((3, 4), 16) == 12
    assert og.host_units(0.25, 12) == 3
    assert og.host_units(0.33, 6) == 2
    # Sweep k/20: exact integer ceiling, never a float artefact (0.15 * 20 = 3 exactly).
    for n in (16, 96, 64, 448):
        for k in range(21):
            assert og.host_units(Fraction(k, 20), n) == -(-k * n // 20)
            assert og.host_units(k / 20, n) == -(-k * n // 20)
    with pytest.raises(ValueError):
        og.host_units(1.5, 4)


def test_split_rows_rejects_ragged_and_overflow():
    A = np.zeros((100, 8))
    with pytest.raises(ValueError):
        og.split_rows(A, 64, 1)
    with pytest.raises(ValueError):
        og.split_rows(np.zeros((128, 8)), 64, 3)


def test_normwise_error():
    ref = np.array([[1.0, -4.0, 2.0]])
    assert og.normwise_error(ref, ref) == 0.0
    assert og.normwise_error(ref + np.array([[0.0, 0.04, 0.0]]), ref) == pytest.approx(0.01)
    assert og.normwise_error(np.zeros((1, 0)), np.zeros((1, 0))) == 0.0
    assert math.isinf(og.normwise_error(np.ones(2), np.zeros(2)))


def test_bf16_widening_is_exact():
    t = synth.normal_bf16((1000,), 0.02, __import__("torch").Generator().manual_seed(0))
    w = og.to_f64(t)
    # every widened value is representable in 8 significant bits
    m, e = np.frexp(w)
    assert np.all(np.abs(m * 256 - np.round(m * 256)) == 0)
