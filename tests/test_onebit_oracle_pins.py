"""Pins of the OneBit oracle (oracle/onebit.py; M8.8 "Native Binary and
Ternary Transformers", 0x06A-0x06B): the sign rule at signed zeros, the FP16
rounding of x * g, the roles of g and h through the SVID identity (a weight
that is exactly sign times a rank-one magnitude is reproduced by scaling the
input by b and the output by a), brute force on a tiny layer, and the
LayerNorm's closed forms over the output dimension."""
import numpy as np

from oracle import onebit


def test_sign_rule():
    w = np.array([[0.0, -0.0, 1e-8, -1e-8, 3.0, -2.0]], np.float32)
    assert onebit.signs(w).tolist() == [[1, 1, 1, -1, 1, -1]]


def test_scaled_input_rounds_once_to_fp16():
    """(1 + 2^-10)^2 = 1 + 2^-9 + 2^-20: the last term is below half an FP16
    ulp at 1 (2^-11) and is dropped; 3 * 0.5 is exact."""
    x = np.array([[1 + 2.0 ** -10, 3.0]], np.float16)
    g = np.array([1 + 2.0 ** -10, 0.5], np.float16)
    xg = onebit.scaled_input(x, g)
    assert xg.dtype == np.float16 and xg.tolist() == [[1 + 2.0 ** -9, 1.5]]


def test_svid_identity():
    """0x06B: W = S * (a b^T) elementwise.  Then x W^T = ((x * b) S^T) * a:
    g = b scales the input columns and h = a the output rows.  Dyadic values
    keep every FP16 product exact, so the two agree to binary64 rounding."""
    rng = np.random.default_rng(0)
    n, k, t = 24, 40, 3
    s = np.where(rng.random((n, k)) < 0.5, 1, -1).astype(np.int8)
    a = (rng.integers(1, 16, n) / 8.0).astype(np.float16)
    b = (rng.integers(1, 16, k) / 16.0).astype(np.float16)
    x = (rng.integers(-16, 17, (t, k)) / 4.0).astype(np.float16)
    w = s.astype(np.float64) * np.outer(a.astype(np.float64), b.astype(np.float64))
    ref = x.astype(np.float64) @ w.T
    assert np.allclose(onebit.projection(x, b, s, a), ref, rtol=1e-15, atol=0)
    # swapping the vectors' roles breaks it
    assert not np.allclose(onebit.projection(x, np.resize(a, k), s, np.resize(b, n)), ref)


def test_brute_force_tiny_layer():
    x = np.array([[1.0, -2.0, 0.5]], np.float16)
    g = np.array([2.0, 0.25, 4.0], np.float16)
    s = np.array([[1, -1, 1], [-1, -1, 1]], np.int8)
    h = np.array([0.5, 2.0], np.float16)
    # x * g = [2, -0.5, 2]; rows: 2 + 0.5 + 2 = 4.5 and -2 + 0.5 + 2 = 0.5
    p = onebit.projection(x, g, s, h)
    assert p.tolist() == [[2.25, 1.0]]
    y = onebit.onebit_linear(x, g, s, h)
    # two outputs: mean 1.625, deviations +-0.625, variance 0.390625
    assert np.allclose(y, [[0.625 / np.sqrt(0.390625 + 1e-5), -0.625 / np.sqrt(0.390625 + 1e-5)]], rtol=1e-14)


def test_layer_norm_over_outputs():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 64)).astype(np.float16)
    g = (1 + 0.1 * rng.standard_normal(64)).astype(np.float16)
    h = (0.5 + rng.random(96)).astype(np.float16)
    s = onebit.signs(rng.standard_normal((96, 64)))
    y = onebit.onebit_linear(x, g, s, h)
    assert y.shape == (5, 96)
    assert np.allclose(y.mean(axis=1), 0, atol=1e-12) and np.allclose(y.var(axis=1), 1, atol=1e-3)
