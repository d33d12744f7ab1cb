"""Pins of the BitNet v1 oracle (oracle/bitnet_v1.py; M8.8 "Native Binary and
Ternary Transformers", 0x02B-0x02E): hand-worked centered codes and their
invariants, the motivation the section gives for centering (a shifted latent
distribution no longer collapses to one sign), hand-worked Q_b = 128 codes
with the encoder epsilon, per-token against per-tensor scales, the rejected
rows, and closed forms of the sub-layer norm."""
import math

import numpy as np
import pytest

import oracle
from oracle import bitnet_v1 as v1


def test_centered_codes_worked_example():
    """Mean 0.375 of [0.125, 0.25, 0.375, 0.75]: below -> -1, the tie -> -1,
    above -> +1; shifting by a dyadic constant keeps every code."""
    w = np.array([[0.125, 0.25, 0.375, 0.75]], np.float32)
    assert v1.centered_binary_codes(w).tolist() == [[-1, -1, -1, 1]]
    assert v1.centered_binary_codes(w + np.float32(3.0)).tolist() == [[-1, -1, -1, 1]]
    assert v1.centered_binary_codes(np.full((2, 3), 0.5, np.float32)).tolist() == [[-1] * 3] * 2


def test_centered_codes_domains():
    """Row 0 = [0, 0, 0, 4] (mean 1), row 1 = [10, 11, 12, 13] (mean 11.5);
    over the whole tensor the mean is 6.25."""
    w = np.array([[0, 0, 0, 4], [10, 11, 12, 13]], np.float32)
    assert v1.centered_binary_codes(w, "row").tolist() == [[-1, -1, -1, 1], [-1, -1, 1, 1]]
    assert v1.centered_binary_codes(w, "tensor").tolist() == [[-1, -1, -1, -1], [1, 1, 1, 1]]
    # groups of 2 columns: [0, 0] -> tie, [0, 4] -> mean 2, [10, 11] -> 10.5, [12, 13] -> 12.5
    assert v1.centered_binary_codes(w, "group", 2).tolist() == [[-1, -1, -1, 1], [-1, 1, -1, 1]]


def test_centering_keeps_a_shifted_distribution_balanced():
    """0x02B: subtracting the mean keeps a shifted latent distribution from
    collapsing to one sign.  N(5, 1) weights: the plain sign rule gives +1
    everywhere, the centered rule about half +1."""
    w = (5.0 + np.random.default_rng(0).standard_normal((64, 256))).astype(np.float32)
    plain, _ = oracle.weight_codes(w, "binary", "tensor")
    centered = v1.centered_binary_codes(w, "tensor")
    assert (plain == 1).all()
    assert 0.45 < (centered == 1).mean() < 0.55


def test_domain_mean_is_sequential_binary64():
    """Values whose fp32 sum loses the small terms: 2^24 then 1s; binary64
    keeps them, so the mean is (2^24 + 4) / 5 rounded once."""
    vals = np.array([2.0 ** 24, 1, 1, 1, 1], np.float32)
    assert v1.domain_mean(vals) == np.float32((2.0 ** 24 + 4) / 5)


def test_act_codes_worked_example():
    """gamma = 1, d = fp32(1 + 1e-5): 128 / d = 127.9987 -> 128 -> clamp 127;
    -64 / d -> -64; 32 / d -> 32; -128 / d = -127.9987 -> -128 (kept: the
    range is [-128, 127]); s_x = 1 / 128."""
    x = np.array([[1.0, -0.5, 0.25, 0.0], [-1.0, 0.5, 0.0, 0.0]], np.float32)
    q, sx, rs = v1.act_quant_v1(x)
    assert q.tolist() == [[127, -64, 32, 0], [-128, 64, 0, 0]]
    assert sx.tolist() == [1 / 128, 1 / 128] and rs.tolist() == [0, 0]
    q0, _, _ = v1.act_quant_v1(x, eps=0.0)
    assert q0.tolist() == [[127, -64, 32, 0], [-128, 64, 0, 0]]


def test_per_token_against_per_tensor():
    """Rows [1, 0.5] and [0.25, 0.125]: one tensor scale gamma = 1 codes the
    second row 32, 16; its own scale 0.25 codes it 127 (128 clamped), 64."""
    x = np.array([[1.0, 0.5], [0.25, 0.125]], np.float32)
    qt, sxt, _ = v1.act_quant_v1(x, per_tensor=True)
    qr, sxr, _ = v1.act_quant_v1(x, per_tensor=False)
    assert qt.tolist() == [[127, 64], [32, 16]] and sxt.tolist() == [1 / 128, 1 / 128]
    assert qr.tolist() == [[127, 64], [127, 64]] and sxr.tolist() == [1 / 128, 0.25 / 128]


def test_act_edge_rows():
    x = np.zeros((4, 8), np.float32)
    x[1, 3] = np.nan
    x[2, 0] = np.float32(3e37)          # 3e37 * 128 overflows fp32
    x[3] = np.float32(2.0 ** -140)      # tiny: d = eps dominates
    q, sx, rs = v1.act_quant_v1(x)
    assert rs.tolist() == [0, 1, 2, 0]
    assert not q[:3].any() and sx[0] == 0 and np.isnan(sx[1:3]).all()
    assert not q[3].any() and sx[3] == np.float32(2.0 ** -147)
    qt, sxt, rst = v1.act_quant_v1(x, per_tensor=True)
    assert not qt.any() and np.isnan(sxt).all() and (rst == 1).all()      # the NaN decides
    qo, sxo, rso = v1.act_quant_v1(x[[0, 2]], per_tensor=True)
    assert not qo.any() and np.isnan(sxo).all() and (rso == 2).all()      # finite, but 128 gamma overflows
    # a zero row with eps = 0: zero codes and output, not 0 / 0
    qz, sxz, rsz = v1.act_quant_v1(np.zeros((2, 4), np.float32), eps=0.0)
    assert not qz.any() and sxz.tolist() == [0.0, 0.0] and rsz.tolist() == [0, 0]


@pytest.mark.parametrize("seed", [0, 1])
def test_layer_norm_closed_forms(seed):
    """Mean 0 and variance var / (var + eps) per row; invariant to adding a
    constant; [1, 2, 3, 4] -> (x - 2.5) / sqrt(1.25 + eps)."""
    x = np.random.default_rng(seed).standard_normal((5, 96)) * 3 + 7
    y = v1.layer_norm(x)
    var = x.var(axis=1)
    assert np.allclose(y.mean(axis=1), 0, atol=1e-12)
    assert np.allclose((y ** 2).mean(axis=1), var / (var + v1.LN_EPS), rtol=1e-12)
    assert np.allclose(v1.layer_norm(x + 100.0), y, atol=1e-9)
    r = v1.layer_norm(np.array([[1.0, 2.0, 3.0, 4.0]]))
    assert np.allclose(r, (np.array([1, 2, 3, 4]) - 2.5) / math.sqrt(1.25 + 1e-5), rtol=1e-15)
    g, b = np.linspace(0.5, 2, 96), np.linspace(-1, 1, 96)
    assert np.allclose(v1.layer_norm(x, gain=g, bias=b), y * g + b, rtol=1e-14)


def test_forward_by_hand():
    """A 2 x 4 binary layer: W rows [0.5, -0.25, 0.25, 1.0] and
    [0, 0.125, -0.5, 0.5] (tensor mean 0.203125); x = [1, -0.5, 0.25, 0]
    -> codes [127, -64, 32, 0]; row codes [+1, -1, +1, +1], [-1, -1, -1, +1];
    acc = 127 + 64 + 32 = 223 and -127 + 64 - 32 = -95; y = acc * beta / 128
    with beta = mean |W| = 3.125 / 8."""
    w = np.array([[0.5, -0.25, 0.25, 1.0], [0.0, 0.125, -0.5, 0.5]], np.float32)
    codes = v1.centered_binary_codes(w, "tensor")
    assert codes.tolist() == [[1, -1, 1, 1], [-1, -1, -1, 1]]
    q, sx, _ = v1.act_quant_v1(np.array([[1.0, -0.5, 0.25, 0.0]], np.float32))
    _, beta = oracle.weight_codes(w, "binary", "tensor")
    acc = q.astype(np.int64) @ codes.T.astype(np.int64)
    assert acc.tolist() == [[223, -95]]
    assert beta[0] == np.float32(3.125 / 8)
    assert np.allclose(acc * (beta[0] * sx[0]), [[223 * 3.125 / 8 / 128, -95 * 3.125 / 8 / 128]], rtol=1e-7)
