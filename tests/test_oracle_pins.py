"""Pins of the CPU oracle against facts the pages and the mathematics fix.

Each test names the passage it checks.  None of them re-types the oracle's own
formula: they use worked values from the pages, hand-derived fixtures, closed
forms, invariants, brute-force add/sub/skip loops, library routines the pages'
reference packer is defined by (numpy.packbits), and exact rational arithmetic.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests.conftest import GOLDEN
from workloads import latent_weights, random_case


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------- ternary codes

def test_ternary_worked_thresholds():
    """M8.8 0x05A/0x05B: absmean 0.5 gives thresholds +-0.25, ties -> 0."""
    g = _golden("ternary_threshold_example.json")
    w = np.array([g["weights"]], np.float32)
    codes, scales = oracle.weight_codes(w, "ternary", "tensor")
    assert scales[0] == np.float32(g["absmean"])
    assert codes[0].tolist() == g["codes"]
    assert (scales[0] * codes[0].astype(np.float32)).tolist() == g["dequantized"]
    # one ulp above the threshold goes to +-1, one ulp below to 0; the row is
    # built so that the absmean stays exactly 0.5 (|u| + |v| = 0.5 exactly)
    t = np.float32(g["threshold"])
    u = np.nextafter(t, np.float32(1))          # 0.25 + 2^-25
    v = np.nextafter(t, np.float32(0))          # 0.25 - 2^-26
    v = np.float32(0.5) - u                     # exact: 0.25 - 2^-25
    w2 = np.array([[u, -v, 0.75, 0.5, -0.5, 0.5, 0.5, -0.75]], np.float32)
    c2, s2 = oracle.weight_codes(w2, "ternary", "tensor")
    assert s2[0] == np.float32(0.5)
    assert c2[0].tolist() == [1, 0, 1, 1, -1, 1, 1, -1]


def test_ternary_gaussian_occupancy_closed_form():
    """M8.8 0x05A dead zone |w| <= s/2 with s = E|w|: for N(0, sigma) latents
    s -> sigma*sqrt(2/pi) and P(code 0) -> erf(1/(2 sqrt(pi))) ~ 0.3101
    (the 'roughly 1/3 zeros' of the ternary decode workload)."""
    w = latent_weights(99, 0, 0, 2048, 2048)
    codes, scales = oracle.weight_codes(w, "ternary", "tensor")
    n = w.size
    sigma = float(np.float32(0.02))
    s_expect = sigma * math.sqrt(2 / math.pi)
    se_s = sigma * math.sqrt(1 - 2 / math.pi) / math.sqrt(n)
    assert abs(float(scales[0]) - s_expect) < 6 * se_s + 1e-9
    p0 = math.erf(1 / (2 * math.sqrt(math.pi)))
    assert abs(p0 - 0.3101) < 1e-4
    frac0 = float((codes == 0).mean())
    assert abs(frac0 - p0) < 6 * math.sqrt(p0 * (1 - p0) / n) + 2e-3  # s is estimated, not exact
    # symmetric +-1 occupancy
    fp, fm = float((codes == 1).mean()), float((codes == -1).mean())
    assert abs(fp - fm) < 5e-3


def test_ternary_scale_is_exact_mean_on_dyadic_values():
    """Scale = mean |W| (M8.8 0x05A).  Dyadic inputs make every partial sum
    exact, so the result must equal the exact rational mean."""
    rng = np.random.default_rng(5)
    w = (rng.integers(-64, 65, size=(7, 48)) / 64.0).astype(np.float32)
    codes, scales = oracle.weight_codes(w, "ternary", "tensor")
    exact = sum(Fraction(abs(float(v))) for v in w.ravel()) / w.size
    assert scales[0] == np.float32(float(exact))
    # per-row and per-group domains
    _, srow = oracle.weight_codes(w, "ternary", "row")
    for r in range(w.shape[0]):
        assert srow[r] == np.float32(float(sum(Fraction(abs(float(v))) for v in w[r]) / w.shape[1]))
    _, sg = oracle.weight_codes(w, "ternary", "group", 20)   # groups 20, 20, 8
    assert sg.shape == (7, 3)
    for r in range(w.shape[0]):
        for gi, (c0, c1) in enumerate([(0, 20), (20, 40), (40, 48)]):
            ex = sum(Fraction(abs(float(v))) for v in w[r, c0:c1]) / (c1 - c0)
            assert sg[r, gi] == np.float32(float(ex))


def test_zero_domain_gives_zero_codes():
    """M8.8 0x09C: a zero weight scale requires zero codes."""
    w = np.zeros((3, 40), np.float32)
    w[1, 5] = 0.3
    codes, sg = oracle.weight_codes(w, "ternary", "group", 16)
    assert sg[0].tolist() == [0.0, 0.0, 0.0] and sg[1, 1] == 0.0 and sg[1, 0] > 0
    assert (codes[0] == 0).all() and codes[1, 5] == 1 and (codes[1, 16:] == 0).all()
    c4, s4 = oracle.weight_codes(w, "int4", "row")
    assert s4[0] == 0 and (c4[0] == 0).all() and c4[1, 5] == 7


def test_nonfinite_weights_rejected():
    w = np.ones((2, 8), np.float32)
    w[1, 3] = np.nan
    with pytest.raises(oracle.OracleError):
        oracle.weight_codes(w, "ternary", "tensor")
    w[1, 3] = np.inf
    with pytest.raises(oracle.OracleError):
        oracle.weight_codes(w, "binary", "row")


# --------------------------------------------------------------- binary codes

def test_binary_total_sign_rule():
    """M8.8 0x06E: +1 if w >= 0 (either signed zero) else -1."""
    w = np.array([[0.0, -0.0, 1e-30, -1e-30, 3.0, -2.5, np.float32(1e-45), -np.float32(1e-45)]], np.float32)
    codes, s = oracle.weight_codes(w, "binary", "row")
    assert codes[0].tolist() == [1, 1, 1, -1, 1, -1, 1, -1]
    assert s[0] == np.float32(float(sum(Fraction(abs(float(v))) for v in w[0]) / 8))


def _words_to_row_stream(packed, fmt, n, k):
    """Gather the packed words back into per-row order by the documented
    offset rule (the word order is this library's own; the test only needs the
    bit order *within* words, which the page fixes)."""
    lay = oracle.layout(fmt, n, k)
    wpl, steps, sk = lay["wpl"], lay["n_steps"], lay["step_k"]
    cpw = 32
    kb = 128
    words = packed.view(np.uint32)
    out = np.zeros((n, steps * sk // 32), np.uint32)
    for r in range(n):
        for s in range(steps):
            for g in range(4):
                for w in range(wpl):
                    src = (((r // 16 * steps + s) * 4 + g) * 16 + r % 16) * wpl + w
                    kpos = s * sk + w * kb + g * (kb // 4)
                    out[r, kpos // cpw] = words[src]
    return out.view(np.uint8)


def test_binary_pack_matches_page_reference_packer():
    """M8.8 0x06E: bits = (1 - s) / 2 packed little-bit-first (numpy.packbits
    with bitorder='little'); unused tail bits zero.  Within each 32-bit word
    the packed artifact keeps exactly that bit order."""
    rng = np.random.default_rng(1)
    for n, k in ((5, 1), (5, 7), (3, 8), (17, 9), (2, 63), (4, 192), (3, 200), (1, 300)):
        s = rng.choice(np.array([-1, 1], np.int8), size=(n, k))
        ref = np.packbits(((1 - s.astype(np.int8)) // 2).astype(np.uint8), axis=1, bitorder="little")
        got = oracle.pack(s, "binary")
        stream = _words_to_row_stream(got, "binary", n, k)
        assert (stream[:, :ref.shape[1]] == ref).all()
        assert (stream[:, ref.shape[1]:] == 0).all()
        assert (oracle.unpack(got, "binary", n, k) == s).all()


def test_binary_unpack_rejects_noncanonical_padding():
    s = np.ones((2, 9), np.int8)
    p = oracle.pack(s, "binary")
    p[1] |= 0x80                      # a tail bit past k = 9
    with pytest.raises(oracle.OracleError):
        oracle.unpack(p, "binary", 2, 9)
    p2 = oracle.pack(s, "binary")
    p2[2 * 4] |= 0x01                 # row 2 of the tile is padding (n = 2)
    with pytest.raises(oracle.OracleError):
        oracle.unpack(p2, "binary", 2, 9)
    with pytest.raises(oracle.OracleError):
        oracle.pack(np.zeros((1, 4), np.int8), "binary")   # zero is not binary


# --------------------------------------------------------------- int4 codes

def test_int4_levels_and_row_max():
    """T4NT model card: symmetric 15 levels -7..+7, all of them used on
    Gaussian weights of its shapes; the row maximum maps to +-7."""
    w = latent_weights(98, 0, 0, 3584, 1280)
    codes, s = oracle.weight_codes(w, "int4", "row", tanh_premap=True)
    assert codes.min() >= -7 and codes.max() <= 7
    assert sorted(np.unique(codes).tolist()) == list(range(-7, 8))
    arg = np.abs(w).argmax(axis=1)
    assert (np.abs(codes[np.arange(w.shape[0]), arg]) == 7).all()
    # premap is tanh(w/3)*3, monotone, so the row max maps to 3 tanh(max/3);
    # it is ~identity here: relative shrink of the max ~ max^2 / 27 (< 3e-4)
    m = np.abs(w.astype(np.float64)).max(axis=1)
    assert np.allclose(s.astype(np.float64), 3 * np.tanh(m / 3) / 7, rtol=3e-7)
    assert (np.abs(s / (m / 7) - 1) < m**2 / 27 * 1.01 + 1e-6).all()


def test_tanh_premap_bounds():
    """T4NT model card: tanh(w/3)*3 keeps 100 % of weights within [-3, 3]."""
    w = np.array([[1e6, -1e6, 40.0, -3.0, 0.02, -1e-3, 0.0, 2.9]], np.float32)
    codes, s = oracle.weight_codes(w, "int4", "row", tanh_premap=True)
    # the largest mapped value is 3 * tanh(big) = 3.0 exactly in fp32
    assert s[0] == np.float32(3.0) / np.float32(7.0)
    mapped = [3 * math.tanh(v / 3) for v in w[0].astype(np.float64)]
    assert all(abs(v) <= 3.0 for v in mapped)
    expect = [max(-7, min(7, round(float(np.float32(v)) / float(s[0])))) for v in mapped]
    # round() in Python is half-to-even, but no value here is a tie
    assert codes[0].tolist() == expect


def test_int4_ties_round_half_even():
    w = np.array([[7.0, 6.5, 5.5, -6.5, -0.5, 0.5, 1.5, 2.5]], np.float32)  # max 7 -> s = 1
    codes, s = oracle.weight_codes(w, "int4", "row")
    assert s[0] == 1.0
    assert codes[0].tolist() == [7, 6, 6, -6, 0, 0, 2, 2]


# ------------------------------------------------------------ layouts / pack

def test_layout_golden_bytes():
    g = _golden("layout_examples.json")
    for case in g["cases"]:
        n, k, fmt = case["n"], case["k"], case["fmt"]
        lay = oracle.layout(fmt, n, k)
        assert (lay["wpl"], lay["n_steps"], lay["packed_bytes"]) == (case["wpl"], case["n_steps"], case["packed_bytes"])
        if fmt == "binary":
            codes = np.ones((n, k), np.int8)
            for r, c in case["minus_ones"]:
                codes[r, c] = -1
        else:
            codes = np.zeros((n, k), np.int8)
            for r, c, v in case["codes"]:
                codes[r, c] = v
        p = oracle.pack(codes, fmt)
        expect = np.zeros(case["packed_bytes"], np.uint8)
        for off, v in case["bytes"].items():
            expect[int(off)] = v
        assert (p == expect).all(), fmt
        assert (oracle.unpack(p, fmt, n, k) == codes).all()
    sc = g["scales"]
    nat = np.zeros((sc["n"], sc["groups"]), np.float32)
    nat[sc["row"], sc["group"]] = 5.0
    packed = oracle.pack_scales(nat, "group", sc["n"], sc["groups"] * 64, 64)
    assert packed.size == sc["size"] and packed[sc["index"]] == 5.0 and packed.sum() == 5.0
    assert (oracle.unpack_scales(packed, "group", sc["n"], sc["groups"] * 64, 64) == nat).all()


@pytest.mark.parametrize("fmt,lo,hi", [("ternary", -1, 1), ("int4", -7, 7), ("binary", -1, 1)])
def test_pack_roundtrip_random(fmt, lo, hi):
    rng = np.random.default_rng(3)
    for n, k in ((1, 1), (4, 3), (17, 15), (3, 16), (33, 17), (5, 100), (2, 257), (16, 1024), (20, 1300)):
        c = rng.integers(lo, hi + 1, size=(n, k)).astype(np.int8)
        if fmt == "binary":
            c[c == 0] = 1
        p = oracle.pack(c, fmt)
        assert p.size == oracle.layout(fmt, n, k)["packed_bytes"]
        assert (oracle.unpack(p, fmt, n, k) == c).all()
        # every code occupies its own field: flipping one code changes the packing
        c2 = c.copy()
        c2[n // 2, k // 2] = -c2[n // 2, k // 2] if c2[n // 2, k // 2] != 0 else 1
        assert (oracle.pack(c2, fmt) != p).sum() >= 1


def test_layout_step_choice():
    """wpl is the widest step that adds no padding beyond the smallest step."""
    assert oracle.layout("ternary", 1, 2560)["wpl"] == 4       # 2560 = 10 x 256
    assert oracle.layout("ternary", 1, 192)["wpl"] == 1        # 192 = 3 x 64, not a multiple of 128
    assert oracle.layout("ternary", 1, 9728)["wpl"] == 4
    assert oracle.layout("binary", 1, 192)["wpl"] == 2         # both 128 and 256 pad 192 to 256
    assert oracle.layout("binary", 1, 768)["wpl"] == 2
    assert oracle.layout("int4", 1, 1280)["wpl"] == 4
    assert oracle.layout("int4", 1, 20)["wpl"] == 2
    for fmt, bits in (("ternary", 2), ("int4", 4), ("binary", 1)):
        lay = oracle.layout(fmt, 32, 4096)
        assert lay["packed_bytes"] * 8 == 32 * 4096 * bits      # no padding when shapes align


def test_reserved_patterns_and_tails_rejected():
    """M8.8 0x0BB: pack/unpack preserves valid symbols, reserved patterns reject."""
    c = np.zeros((1, 16), np.int8)
    p = oracle.pack(c, "ternary")
    p[2] = 0b10                           # ternary field 10 is reserved
    with pytest.raises(oracle.OracleError):
        oracle.unpack(p, "ternary", 1, 16)
    p4 = oracle.pack(np.zeros((1, 8), np.int8), "int4")
    p4[1] = 0x08                          # int4 nibble 1000 (-8) is reserved
    with pytest.raises(oracle.OracleError):
        oracle.unpack(p4, "int4", 1, 8)
    pt = oracle.pack(np.ones((1, 5), np.int8), "ternary")
    pt[3] |= 0x40                         # field of k = 15 > 5: noncanonical tail
    with pytest.raises(oracle.OracleError):
        oracle.unpack(pt, "ternary", 1, 5)
    with pytest.raises(oracle.OracleError):
        oracle.pack(np.full((1, 4), 2, np.int8), "ternary")
    with pytest.raises(oracle.OracleError):
        oracle.pack(np.full((1, 4), -8, np.int8), "int4")


# ---------------------------------------------------- activation quantisation

def test_act_quant_golden():
    """M8.8 0x02C/0x05C worked by hand: ties to even, 127-based scale."""
    for row in _golden("act_quant_examples.json")["rows"]:
        x = np.array([row["x"]], np.float32)
        q, sx, st = oracle.act_quant(x)
        assert st[0] == 0
        assert q[0].tolist() == row["q"]
        if "sx" in row:
            assert sx[0] == np.float32(row["sx"])
        if "sx_bits" in row:
            assert int(sx.view(np.uint32)[0]) == row["sx_bits"]


def test_act_quant_invariants():
    """Per-token absmax (M8.8 0x05C): the row max maps to exactly +-127; codes
    are odd under x -> -x; scaling a row by a power of two leaves the codes and
    scales the step exactly; rows are independent (per-token scale broadcast,
    M8.8 0x0BB)."""
    _, x = random_case(11, 1, 300, 64)
    x[3] = 0.0
    q, sx, st = oracle.act_quant(x)
    assert (st == 0).all()
    nz = np.abs(x).max(axis=1) > 0
    assert (np.abs(q[nz]).max(axis=1) == 127).all()
    am = np.abs(x).argmax(axis=1)
    assert (np.abs(q[np.arange(64), am])[nz] == 127).all()
    assert (q[3] == 0).all() and sx[3] == 0
    qn, sxn, _ = oracle.act_quant(-x)
    assert (qn == -q).all() and (sxn == sx).all()
    for p in (0.25, 2.0, 1024.0):
        q2, sx2, _ = oracle.act_quant(x * np.float32(p))
        assert (q2 == q).all() and (sx2 == sx * np.float32(p)).all()
    # independence of rows: changing row 5 leaves every other row unchanged
    x2 = x.copy()
    x2[5] *= np.float32(3.0)
    q3, sx3, _ = oracle.act_quant(x2)
    keep = np.arange(64) != 5
    assert (q3[keep] == q[keep]).all() and (sx3[keep] == sx[keep]).all()
    # reconstruction error at most half a step
    rec = q.astype(np.float64) * sx.astype(np.float64)[:, None]
    assert (np.abs(rec - x) <= 0.5 * sx.astype(np.float64)[:, None] * (1 + 1e-6) + 1e-30).all()


def test_act_quant_integer_identity():
    """Inputs already on the int8 grid with max |x| = 127: scale 1, q == x."""
    rng = np.random.default_rng(2)
    x = rng.integers(-127, 128, size=(9, 77)).astype(np.float32)
    x[:, 0] = 127.0
    q, sx, st = oracle.act_quant(x)
    assert (q == x.astype(np.int8)).all() and (sx == 1.0).all() and (st == 0).all()


def test_act_quant_rejects_bad_rows():
    x = np.ones((4, 5), np.float32)
    x[1, 2] = np.nan
    x[2, 0] = np.inf
    x[3] = np.float32(1e-45)          # 127 / m overflows fp32
    q, sx, st = oracle.act_quant(x)
    assert st.tolist() == [0, oracle.ROW_NONFINITE, oracle.ROW_NONFINITE, oracle.ROW_OVERFLOW]
    assert (q[1:] == 0).all() and np.isnan(sx[1:]).all()


# ------------------------------------------------------------ integer product

def _brute_add_sub(q, codes):
    """Atomic-1Bit README definition: w = +1 adds, w = -1 subtracts, w = 0 skips;
    general codes (int4) add |w| copies with the code's sign."""
    t, k = q.shape
    n = codes.shape[0]
    out = [[0] * n for _ in range(t)]
    for i in range(t):
        for r in range(n):
            acc = 0
            for c in range(k):
                w = int(codes[r, c])
                a = int(q[i, c])
                for _ in range(abs(w)):
                    acc = acc + a if w > 0 else acc - a
            out[i][r] = acc
    return np.array(out, np.int64)


def test_add_sub_skip_identity():
    """Atomic-1Bit README: a row with one +1 returns that activation, one -1 its
    negation, all zeros returns 0 (M8.8 0x05D partition into P+ and P-)."""
    _, x = random_case(4, 1, 37, 3)
    q, sx, _ = oracle.act_quant(x)
    k = 37
    codes = np.zeros((2 * k + 1, k), np.int8)
    for j in range(k):
        codes[j, j] = 1
        codes[k + j, j] = -1
    acc = oracle.int_matmul(q, codes)[:, :, 0]
    assert (acc[:, :k] == q.astype(np.int64)).all()
    assert (acc[:, k:2 * k] == -q.astype(np.int64)).all()
    assert (acc[:, 2 * k] == 0).all()
    # binary all +1 gives the row sum
    ones = np.ones((1, k), np.int8)
    assert (oracle.int_matmul(q, ones)[:, 0, 0] == q.astype(np.int64).sum(axis=1)).all()


@pytest.mark.parametrize("fmt,lo,hi", [("ternary", -1, 1), ("int4", -7, 7)])
def test_int_matmul_brute_force(fmt, lo, hi):
    """Brute force on tiny non-square shapes (catches transposed operands)."""
    rng = np.random.default_rng(7)
    for (t, n, k) in [(1, 1, 1), (2, 3, 5), (3, 5, 17), (4, 2, 33)]:
        q = rng.integers(-127, 128, size=(t, k)).astype(np.int8)
        c = rng.integers(lo, hi + 1, size=(n, k)).astype(np.int8)
        acc = oracle.int_matmul(q, c)
        assert acc.shape == (t, n, 1)
        assert (acc[:, :, 0] == _brute_add_sub(q, c)).all()
        assert (acc[:, :, 0] == q.astype(np.int64) @ c.astype(np.int64).T).all()


def test_group_partials_and_k_sharding():
    """Group partials sum to the whole-row product; splitting K on group
    boundaries and adding int partials is exact (the row-parallel contract,
    M8.8 0x08B/0x08C, checked against its own unsharded reference)."""
    rng = np.random.default_rng(8)
    q = rng.integers(-127, 128, size=(5, 300)).astype(np.int8)
    c = rng.integers(-1, 2, size=(7, 300)).astype(np.int8)
    full = oracle.int_matmul(q, c)[:, :, 0]
    parts = oracle.int_matmul(q, c, 128)
    assert parts.shape == (5, 7, 3)
    assert (parts.sum(axis=2) == full).all()
    shard = sum(oracle.int_matmul(q[:, a:b], c[:, a:b])[:, :, 0] for a, b in [(0, 128), (128, 256), (256, 300)])
    assert (shard == full).all()
    # column (N) sharding: concatenating row blocks equals the whole
    cat = np.concatenate([oracle.int_matmul(q, c[a:b])[:, :, 0] for a, b in [(0, 3), (3, 7)]], axis=1)
    assert (cat == full).all()


def test_acc_bound():
    """M8.8 0x09C: the worst-case dot product must fit INT32."""
    kmax_t = (2**31 - 1) // 127
    assert oracle.acc_bound_ok("ternary", kmax_t) and not oracle.acc_bound_ok("ternary", kmax_t + 1)
    kmax_4 = (2**31 - 1) // (127 * 7)
    assert oracle.acc_bound_ok("int4", kmax_4) and not oracle.acc_bound_ok("int4", kmax_4 + 1)
    big = np.zeros(oracle.layout("int4", 1, kmax_4 + 1)["packed_bytes"], np.uint8)
    with pytest.raises(oracle.OracleError):
        oracle.linear(big, np.ones(1, np.float32), "int4", "tensor", 0, 1, kmax_4 + 1,
                      np.zeros((1, kmax_4 + 1), np.int8), np.ones(1, np.float32))


# ------------------------------------------------------------------ epilogue

def test_epilogue_exact_with_dyadic_scales():
    """y = acc * s_x * s_w (M8.8 0x02D): with power-of-two scales every fp32
    product is exact, so y must equal the exact rational value."""
    acc = np.array([[[12345], [-7]], [[0], [999999]]], np.int64)
    sx = np.array([2.0**-7, 0.5], np.float32)
    sw = np.array([2.0**-6, 4.0], np.float32)
    y32, y64 = oracle.epilogue(acc, sx, sw, "row")
    for i in range(2):
        for r in range(2):
            exact = Fraction(int(acc[i, r, 0])) * Fraction(float(sx[i])) * Fraction(float(sw[r]))
            assert Fraction(float(y32[i, r])) == exact and Fraction(float(y64[i, r])) == exact
    # unit ternary decoder (M8.8 0x05B): scale 1 gives y = acc * s_x
    y1, _ = oracle.epilogue(acc, sx, np.ones(1, np.float32), "tensor")
    assert (y1 == (acc[:, :, 0].astype(np.float32) * sx[:, None])).all()
    # group scales: sum of group partials times their own scale
    accg = np.array([[[3, -5, 7]]], np.int64)
    swg = np.array([[0.5, 0.25, 2.0]], np.float32)
    yg, _ = oracle.epilogue(accg, np.array([0.125], np.float32), swg, "group")
    assert yg[0, 0] == np.float32(0.125 * (1.5 - 1.25 + 14.0))


def test_linear_matches_dense_fp64_reconstruction():
    """The layer equals a dense fp64 matmul of the dequantised operands
    (s_x q)(s_w c)^T - the operator's definition (M8.8 0x09C)."""
    w, x = random_case(21, 37, 300, 6)
    for fmt, scale, group, pre in [("ternary", "tensor", 0, False), ("ternary", "group", 128, False),
                                   ("binary", "row", 0, False), ("int4", "row", 0, True),
                                   ("int4", "group", 64, False), ("binary", "group", 128, False)]:
        packed, psc, codes, sc = oracle.quantize_and_pack(w, fmt, scale, group, pre)
        q, sx, _ = oracle.act_quant(x)
        y32, y64, acc = oracle.linear(packed, psc, fmt, scale, group, 37, 300, q, sx)
        if scale == "group":
            G = sc.shape[1]
            wdq = (codes.astype(np.float64).reshape(37, -1) *
                   np.repeat(sc.astype(np.float64), group, axis=1)[:, :300])
        else:
            wdq = codes.astype(np.float64) * (sc.astype(np.float64).reshape(-1, 1) if scale == "row"
                                              else float(sc[0]))
        dense = (q.astype(np.float64) * sx.astype(np.float64)[:, None]) @ wdq.T
        assert np.allclose(y64, dense, rtol=1e-12, atol=1e-12), fmt
        assert (np.abs(y32 - y64) <= 1e-6 + 1e-5 * np.abs(y64)).all(), fmt
        # the unpacked codes are the quantiser's codes and the product is exact
        assert (acc.sum(axis=2) == q.astype(np.int64) @ codes.astype(np.int64).T).all()
