"""Pins of the split decode-attention oracle (DAK paper §5, batch split of the KV
cache) against closed forms, special cases and a library softmax."""
import numpy as np
import pytest
from scipy.special import softmax as sp_softmax

import synth
from oracle import attention as oa
from oracle.gemm import to_f64


def test_single_position_returns_its_value_row():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((2, 4, 8))
    K = rng.standard_normal((2, 2, 1, 8))
    V = rng.standard_normal((2, 2, 1, 8))
    out = oa.decode_attention(q, K, V, 0.3)
    for b in range(2):
        for j in range(4):
            assert np.array_equal(out[b, j], V[b, j // 2, 0])


def test_equal_keys_give_mean_of_values_exactly():
    # Equal scores -> uniform weights; integer V and a power-of-two context make
    # the mean exact.
    T = 64
    K = np.ones((1, 1, T, 16))
    V = to_f64(synth.int_valued_bf16((1, 1, T, 16), -2, 2, seed=9))
    q = np.full((1, 1, 16), 0.7)
    out = oa.decode_attention(q, K, V, 1.0 / 4.0)
    assert np.array_equal(out[0, 0], V[0, 0].sum(axis=0) / T)


def test_constant_values_are_returned_whatever_the_scores():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 2, 8))
    K = rng.standard_normal((1, 1, 37, 8)) * 5
    V = np.full((1, 1, 37, 8), 0.25)
    out = oa.decode_attention(q, K, V, 1.0)
    assert np.allclose(out, 0.25, rtol=0, atol=1e-15)


def test_dominant_key_selects_its_row():
    D, T = 8, 50
    K = np.zeros((1, 1, T, D))
    K[0, 0, 17, 0] = 1000.0
    q = np.zeros((1, 1, D))
    q[0, 0, 0] = 1.0
    V = np.arange(T * D, dtype=np.float64).reshape(1, 1, T, D)
    out = oa.decode_attention(q, K, V, 1.0)
    assert np.array_equal(out[0, 0], V[0, 0, 17])


def test_two_keys_closed_form_pins_scale_and_sign():
    # Two positions with scores s1 > s2: weight of position 0 is the logistic
    # function of scale * (s1 - s2).
    D = 4
    q = np.array([[[1.0, 0.0, 0.0, 0.0]]])
    K = np.zeros((1, 1, 2, D))
    K[0, 0, 0, 0] = 3.0
    K[0, 0, 1, 0] = 1.0
    V = np.zeros((1, 1, 2, D))
    V[0, 0, 0, 1] = 1.0
    scale = 0.5
    out = oa.decode_attention(q, K, V, scale)
    w0 = 1.0 / (1.0 + np.exp(-scale * (3.0 - 1.0)))
    assert out[0, 0, 1] == pytest.approx(w0, rel=1e-15)
    assert out[0, 0, 0] == 0.0


def test_grouped_query_heads_read_their_kv_head():
    # KV head g holds V == g + 1 everywhere, so query head j must return
    # group(j) + 1 with group(j) = j // (Hq / Hkv) (consecutive heads share).
    Hq, Hkv, T, D = 8, 2, 5, 4
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, Hq, D))
    K = rng.standard_normal((1, Hkv, T, D))
    V = np.stack([np.full((T, D), g + 1.0) for g in range(Hkv)])[None]
    out = oa.decode_attention(q, K, V, 1.0)
    for j in range(Hq):
        assert np.allclose(out[0, j], j // 4 + 1.0, rtol=0, atol=1e-14)
    assert [oa.kv_group(j, 32, 8) for j in (0, 3, 4, 31)] == [0, 0, 1, 7]


def test_matches_library_softmax():
    rng = np.random.default_rng(4)
    T, D = 300, 16
    q = rng.standard_normal((1, 1, D))
    K = rng.standard_normal((1, 1, T, D))
    V = rng.standard_normal((1, 1, T, D))
    scale = 1.0 / np.sqrt(D)
    ref = sp_softmax(scale * (K[0, 0] @ q[0, 0])) @ V[0, 0]
    out = oa.decode_attention(q, K, V, scale)
    assert np.allclose(out[0, 0], ref, rtol=1e-13, atol=1e-15)


def test_batch_split_is_exact():
    q, K, V = synth.attn_inputs(4, 4, 2, 8, 33, seed=1)
    q, K, V = to_f64(q), to_f64(K), to_f64(V)
    ref = oa.decode_attention(q, K, V, 0.35)
    for h in range(5):
        out = oa.split_decode_attention(q, K[:h], V[:h], K[h:], V[h:], 0.35)
        assert np.array_equal(out, ref)


# ---------------------------------------------------------------------------
# Ragged batch: request b attends to its first lens[b] positions only
# ---------------------------------------------------------------------------
def test_ragged_one_valid_position_returns_that_value_row():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((3, 4, 8))
    K = rng.standard_normal((3, 2, 6, 8))
    V = rng.standard_normal((3, 2, 6, 8))
    out = oa.decode_attention_lens(q, K, V, 0.7, [1, 1, 1])
    for b in range(3):
        for j in range(4):
            assert np.array_equal(out[b, j], V[b, j // 2, 0])


def test_ragged_equal_keys_give_the_mean_of_the_valid_rows():
    # All keys equal: every valid position has the same weight 1/lens[b].
    rng = np.random.default_rng(6)
    q = rng.standard_normal((2, 2, 4))
    K = np.ones((2, 1, 9, 4))
    V = rng.integers(-3, 4, size=(2, 1, 9, 4)).astype(np.float64)
    lens = [9, 4]
    out = oa.decode_attention_lens(q, K, V, 0.3, lens)
    for b in range(2):
        assert np.allclose(out[b, :], V[b, 0, :lens[b]].mean(axis=0)[None, :], rtol=0, atol=1e-15)


def test_ragged_positions_past_the_length_do_not_matter():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((2, 4, 8))
    K = rng.standard_normal((2, 2, 10, 8))
    V = rng.standard_normal((2, 2, 10, 8))
    lens = [10, 3]
    a = oa.decode_attention_lens(q, K, V, 0.5, lens)
    K2, V2 = K.copy(), V.copy()
    K2[1, :, 3:] = 100.0
    V2[1, :, 3:] = -7.0
    assert np.array_equal(oa.decode_attention_lens(q, K2, V2, 0.5, lens), a)
    # full lengths are the unragged attention
    assert np.array_equal(oa.decode_attention_lens(q, K, V, 0.5, [10, 10]), oa.decode_attention(q, K, V, 0.5))
    with pytest.raises(ValueError):
        oa.decode_attention_lens(q, K, V, 0.5, [0, 3])
