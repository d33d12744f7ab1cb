"""Pins of the decode-step oracle (oracle/model.py) against closed forms,
invariants and special cases of its definitions (the b1.58 recipe the M8.8
"Native Binary and Ternary Transformers" page names: RMSNorm, rotary position
embeddings, SwiGLU; softmax attention).  None re-types the oracle's formula;
each is chosen so that a plausible slip - a missing gain, mean instead of mean
of squares, the wrong pairing or sign of a rotation, an unscaled or unnormalised
softmax, a sigmoid in place of SiLU - fails at least one of them."""
import math

import numpy as np
import pytest

import oracle
from oracle import model as om


# ----------------------------------------------------------------- RMSNorm

def test_rmsnorm_constant_row_closed_form():
    """x = c * 1: mean(x^2) = c^2, so the output is c / sqrt(c^2 + eps) * g."""
    d = 16
    g = np.arange(1, d + 1, dtype=np.float64) / 8
    for c in (3.0, -0.5, 1e-4):
        y = om.rmsnorm(np.full(d, c), g, eps=1e-6)
        assert np.allclose(y, c / math.sqrt(c * c + 1e-6) * g, rtol=1e-14, atol=0)


def test_rmsnorm_unit_rms_and_scale_invariance():
    """With g = 1 and eps = 0 the output has root mean square 1 and does not
    change when x is scaled by a positive factor; g multiplies elementwise."""
    rng = np.random.default_rng(0)
    x = rng.standard_normal(256)
    y = om.rmsnorm(x, np.ones(256), eps=0.0)
    assert abs(math.sqrt(np.mean(y * y)) - 1.0) < 1e-14
    assert np.allclose(om.rmsnorm(7.5 * x, np.ones(256), eps=0.0), y, rtol=1e-13, atol=0)
    g = rng.standard_normal(256)
    assert np.allclose(om.rmsnorm(x, g, eps=0.0), y * g, rtol=1e-13, atol=0)
    # not mean-centred: adding a constant changes the result
    assert not np.allclose(om.rmsnorm(x + 1.0, np.ones(256), eps=0.0), y)


def test_rmsnorm_two_element_worked_value():
    """x = (3, 4): mean of squares 12.5, so y = x / sqrt(12.5) (eps = 0)."""
    y = om.rmsnorm(np.array([3.0, 4.0]), np.ones(2), eps=0.0)
    assert np.allclose(y, [3 / math.sqrt(12.5), 4 / math.sqrt(12.5)], rtol=1e-15, atol=0)


# ----------------------------------------------------------------- rotary

def test_rope_position_zero_is_identity():
    v = np.random.default_rng(1).standard_normal(256)
    assert np.array_equal(om.rope(v, 0, 4), v)


def test_rope_one_pair_is_a_rotation_by_pos_radians():
    """head_dim 2: one pair with frequency base^0 = 1, so position p rotates
    (a, b) by p radians counter-clockwise."""
    a, b = 0.6, -1.3
    for p in (1, 2, 5, 77):
        y = om.rope(np.array([a, b]), p, 1)
        assert np.allclose(y, [a * math.cos(p) - b * math.sin(p), a * math.sin(p) + b * math.cos(p)],
                           rtol=1e-13, atol=1e-15)


def test_rope_pairing_and_frequencies_head_dim_4():
    """head_dim 4: dimensions (0, 2) rotate at frequency 1 and (1, 3) at
    base^(-1/2) = 0.01; a vector with only dimension 1 set stays in the
    (1, 3) plane."""
    p = 3
    y = om.rope(np.array([0.0, 1.0, 0.0, 0.0]), p, 1)
    w = p * 10000.0 ** -0.5
    assert np.allclose(y, [0.0, math.cos(w), 0.0, math.sin(w)], rtol=1e-13, atol=1e-15)
    y = om.rope(np.array([1.0, 0.0, 0.0, 0.0]), p, 1)
    assert np.allclose(y, [math.cos(p), 0.0, math.sin(p), 0.0], rtol=1e-13, atol=1e-15)


def test_rope_preserves_norms_and_depends_on_relative_position():
    """A rotation keeps every pair's length, and q . k after rotation depends
    only on the distance between the two positions (per head)."""
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal(256), rng.standard_normal(256)
    for p in (0, 9, 127):
        r = om.rope(q, p, 4).reshape(4, 2, 32)
        q4 = q.reshape(4, 2, 32)
        assert np.allclose(np.hypot(r[:, 0], r[:, 1]), np.hypot(q4[:, 0], q4[:, 1]), rtol=1e-12)
    def dots(m, n):
        return (om.rope(q, m, 4).reshape(4, 64) * om.rope(k, n, 4).reshape(4, 64)).sum(axis=1)
    assert np.allclose(dots(10, 3), dots(57, 50), rtol=1e-10)
    assert not np.allclose(dots(10, 3), dots(10, 4))


# ----------------------------------------------------------------- attention

def test_attention_single_position_returns_its_value():
    rng = np.random.default_rng(3)
    q, k, v = rng.standard_normal(256), rng.standard_normal((1, 256)), rng.standard_normal((1, 256))
    assert np.allclose(om.attend(q, k, v, 4), v[0], rtol=1e-15, atol=0)


def test_attention_zero_query_averages_the_values():
    """q = 0: every score is 0, the softmax is uniform, the output is the mean
    of the cached values."""
    rng = np.random.default_rng(4)
    k, v = rng.standard_normal((9, 256)), rng.standard_normal((9, 256))
    assert np.allclose(om.attend(np.zeros(256), k, v, 4), v.mean(axis=0), rtol=1e-13, atol=1e-15)


def test_attention_two_keys_logistic_weight_and_scaling():
    """Two positions whose keys differ only in one head: the weight of the
    second is the logistic function of (s1 - s0) with s = q . k / sqrt(64)
    (the 1/sqrt(head_dim) scale); other heads see equal scores."""
    q = np.zeros(256)
    q[0] = 1.0                       # head 0
    k = np.zeros((2, 256))
    k[1, 0] = 4.0                    # score difference 4 / 8 = 0.5 in head 0
    v = np.zeros((2, 256))
    v[0, :] = 1.0
    v[1, :] = 3.0
    out = om.attend(q, k, v, 4)
    w1 = 1.0 / (1.0 + math.exp(-0.5))
    assert np.allclose(out[:64], 1.0 + 2.0 * w1, rtol=1e-14)
    assert np.allclose(out[64:], 2.0, rtol=1e-14)          # heads 1-3: uniform


def test_attention_heads_are_independent():
    rng = np.random.default_rng(5)
    q, k, v = rng.standard_normal(256), rng.standard_normal((6, 256)), rng.standard_normal((6, 256))
    base = om.attend(q, k, v, 4)
    v2 = v.copy()
    v2[:, 64:128] += 10.0
    changed = om.attend(q, k, v2, 4)
    assert np.array_equal(changed[:64], base[:64]) and np.array_equal(changed[128:], base[128:])
    assert np.allclose(changed[64:128], base[64:128] + 10.0, rtol=1e-12)


# ----------------------------------------------------------------- SwiGLU

def test_swiglu_closed_forms():
    """SiLU(0) = 0; SiLU(ln 3) = (3/4) ln 3 (e^-z = 1/3); SiLU(z) -> z for
    large z and -> 0 for very negative z; the up branch multiplies."""
    z = np.array([0.0, math.log(3.0), 40.0, -40.0])
    y = om.swiglu(z, np.ones(4))
    assert y[0] == 0.0
    assert math.isclose(y[1], 0.75 * math.log(3.0), rel_tol=1e-15)
    assert math.isclose(y[2], 40.0, rel_tol=1e-15)
    assert abs(y[3]) < 1e-15
    assert np.allclose(om.swiglu(z, np.full(4, -2.0)), -2.0 * y, rtol=1e-15, atol=0)


# ----------------------------------------------------------------- decode step

def _tiny_model(seed=0, d=16, heads=2, ff=32, vocab=40, layers=2, context=8):
    rng = np.random.default_rng(seed)
    embed = rng.standard_normal((vocab, d)).astype(np.float32)
    norms = (1.0 + 0.1 * rng.standard_normal((2 * layers + 1, d))).astype(np.float32)
    packed, scales = [], []
    shapes = [(3 * d, d), (d, d), (ff, d), (ff, d), (d, ff)] * layers + [(vocab, d)]
    for n, k in shapes:
        w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
        pk, sc, _, _ = oracle.quantize_and_pack(w, "ternary", "tensor")
        packed.append(pk)
        scales.append(sc)
    return om.Model(d, layers, heads, ff, vocab, context, embed, norms, packed, scales)


def test_decode_step_position_zero_structure():
    """At position 0 the rotation is the identity and attention sees one
    position, so the attention output is the value part of the qkv
    projection, the cached key is its key part, and each block adds its two
    branch outputs to the residual stream; the next token is the argmax."""
    m = _tiny_model()
    kc = np.zeros((m.n_layers, m.context, m.d))
    vc = np.zeros_like(kc)
    logits, nxt, tr = om.decode_step(m, 7, 0, kc, vc)
    d = m.d
    assert np.allclose(tr[0]["x_in"], m.embed[7])
    for l, t in enumerate(tr):
        assert np.array_equal(t["attn"], t["qkv"][2 * d:])
        assert np.array_equal(kc[l, 0], t["qkv"][d:2 * d]) and np.array_equal(vc[l, 0], t["qkv"][2 * d:])
        assert np.allclose(t["x_out"], t["x_in"] + t["o"] + t["down"], rtol=1e-15, atol=1e-15)
    assert nxt == int(np.argmax(logits)) and logits.dtype == np.float32


def test_decode_step_is_causal_and_uses_the_cache():
    """Step 1 attends over positions 0 and 1: running step 0 with another
    token changes step 1's result, while step 0's own result does not depend
    on anything after it."""
    m = _tiny_model(1)
    def run(tokens):
        kc = np.zeros((m.n_layers, m.context, m.d))
        vc = np.zeros_like(kc)
        return [om.decode_step(m, t, p, kc, vc)[0] for p, t in enumerate(tokens)]
    a, b = run([3, 5]), run([4, 5])
    c = run([3, 9])
    assert np.array_equal(a[0], c[0])
    assert not np.array_equal(a[1], b[1])
