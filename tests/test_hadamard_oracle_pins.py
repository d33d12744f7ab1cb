"""Pins of the H-BitLinear activation oracle (oracle/hadamard.py; M8.8 "Native
Binary and Ternary Transformers", 0x07C) against the dense definition of the
Walsh-Hadamard transform (scipy.linalg.hadamard, Sylvester order, in
binary64), its algebra (orthonormal, an involution, block-diagonal), the
outlier spreading the section describes, and hand-worked INT4 codes."""
import math

import numpy as np
import pytest
from scipy.linalg import hadamard

from oracle import hadamard as oh


def test_block_size():
    assert [oh.block_size(k) for k in (64, 192, 256, 768, 1024, 1280, 2560, 3584, 4096, 9728, 65536)] == \
        [64, 64, 256, 256, 1024, 256, 512, 512, 2048, 512, 2048]
    assert oh.block_size(32) == 0 and oh.block_size(100) == 0


@pytest.mark.parametrize("b", [64, 256, 512, 2048])
def test_fwht_matches_dense_sylvester_matrix(b):
    """The fast fp32 form equals H_b x / sqrt(b) (dense, binary64) to fp32
    rounding: log2(b) stages of one rounding each, and the final scale."""
    rng = np.random.default_rng(b)
    x = rng.standard_normal((3, 2 * b)).astype(np.float32)
    got = oh.fwht_blocks(x, b).astype(np.float64)
    H = hadamard(b).astype(np.float64) / math.sqrt(b)
    ref = np.concatenate([x[:, :b].astype(np.float64) @ H.T, x[:, b:].astype(np.float64) @ H.T], axis=1)
    tol = (math.log2(b) + 2) * 2.0 ** -24 * np.sqrt(b) * np.abs(x).max()
    assert np.abs(got - ref).max() <= tol


def test_fwht_algebra():
    """Orthonormal (norms kept), an involution (applied twice it returns x),
    block-diagonal (a block's output depends on that block only); the unit
    vector e0 maps to the constant 1 / sqrt(b)."""
    rng = np.random.default_rng(1)
    b = 512
    x = rng.standard_normal((4, 4 * b)).astype(np.float32)
    y = oh.fwht_blocks(x, b)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-5)
    assert np.allclose(oh.fwht_blocks(y, b), x, rtol=0, atol=2e-5 * np.abs(x).max())
    x2 = x.copy()
    x2[:, b:2 * b] *= 3.0
    y2 = oh.fwht_blocks(x2, b)
    assert np.array_equal(y2[:, :b], y[:, :b]) and np.array_equal(y2[:, 2 * b:], y[:, 2 * b:])
    e0 = np.zeros((1, b), np.float32)
    e0[0, 0] = 1.0
    assert np.allclose(oh.fwht_blocks(e0, b), 1.0 / math.sqrt(b), rtol=1e-6)


def test_rotation_spreads_an_outlier():
    """0x07C: the transform spreads concentrated channel outliers.  A row of
    small values with one spike of 100: before, INT4 absmax codes leave every
    other channel at 0; after rotating, max |x'| is about 100 / sqrt(b) and
    most channels keep a nonzero code."""
    rng = np.random.default_rng(2)
    b = 256
    x = (0.5 * rng.standard_normal((1, b))).astype(np.float32)
    x[0, 17] = 100.0
    q_plain, _, _ = oh.act_quant4(x)
    q_rot, sx, _ = oh.rotated_act_quant4(x)
    assert np.count_nonzero(q_plain) == 1
    assert np.count_nonzero(q_rot) > b // 2
    assert abs(sx[0] * 7 - 100 / math.sqrt(b)) < 0.5 * 7 * sx[0]


def test_int4_codes_worked_example():
    """m = 3.5 -> r = 2; x' r = 7, -2, 1, 0.5 (ties to even -> 0), -7, 2.5 (-> 2),
    -6.999..., 0; s_x = 0.5."""
    row = np.array([[3.5, -1.0, 0.5, 0.25, -3.5, 1.25, -3.4999998, 0.0]], np.float32)
    q, sx, rs = oh.act_quant4(row)
    assert q[0].tolist() == [7, -2, 1, 0, -7, 2, -7, 0]
    assert sx[0] == np.float32(0.5) and rs[0] == 0


def test_int4_edge_rows():
    x = np.zeros((4, 64), np.float32)
    x[1, 3] = np.nan
    x[2, 5] = -np.inf
    x[3, :] = np.float32(1e-45)
    q, sx, rs = oh.act_quant4(x)
    assert rs.tolist() == [0, 1, 1, 2]
    assert not q.any() and sx[0] == 0 and np.isnan(sx[1:]).all()
