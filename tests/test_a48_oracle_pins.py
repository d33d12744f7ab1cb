"""Pins of the BitNet a4.8 activation oracle (oracle/a48.py; M8.8 "Native
Binary and Ternary Transformers", 0x07B): the keep mask against brute force
over every subset of tiny rows, hand-worked codes (ties to even in the 4-bit
rule, ties at the threshold in the sparse rule), the reduction to the dense
INT8 quantiser when every entry is kept, sign symmetry, and rejected rows."""
import itertools

import numpy as np
import pytest

import oracle
from oracle import a48


def _brute_mask(row, keep):
    """Among the keep-subsets of largest total |x|, the one whose sorted
    indices come first: the largest magnitudes, ties to the lower index."""
    a = np.abs(row.astype(np.float64))
    best = None
    for sub in itertools.combinations(range(len(row)), keep):
        key = (-a[list(sub)].sum(), sub)
        if best is None or key < best:
            best = key
    m = np.zeros(len(row), bool)
    m[list(best[1])] = True
    return m


@pytest.mark.parametrize("seed", range(6))
def test_keep_mask_brute_force(seed):
    rng = np.random.default_rng(seed)
    k = 8
    rows = [rng.standard_normal(k).astype(np.float32),
            (rng.integers(-3, 4, k) * 0.5).astype(np.float32),       # many equal magnitudes
            np.zeros(k, np.float32)]
    x = np.stack(rows)
    for keep in range(1, k + 1):
        got = a48.keep_mask(x, keep)
        for i, row in enumerate(rows):
            assert (got[i] == _brute_mask(row, keep)).all(), (seed, keep, row)
        assert (got.sum(axis=1) == keep).all()


def test_keep_mask_rejects_bad_keep():
    x = np.ones((1, 4), np.float32)
    for keep in (0, 5):
        with pytest.raises(ValueError):
            a48.keep_mask(x, keep)


def test_input_codes_hand_worked():
    """m = 3.5, 7 / m = 2: codes rint([1, -3.5, 7, 0.5, -0.5]) with ties to
    even = [1, -4, 7, 0, 0]; s_x = 0.5."""
    x = np.array([[0.5, -1.75, 3.5, 0.25, -0.25]], np.float32)
    q, sx, rs = a48.input_codes(x)
    assert q.tolist() == [[1, -4, 7, 0, 0]] and sx.tolist() == [0.5] and rs.tolist() == [0]


def test_sparse_codes_hand_worked():
    """x = [0.1, -3, 2, -2, 0.5]: keep 3 keeps indices 1, 2, 3; fp32(127 / 3)
    = 42.333332, so 2 -> rint(84.666664) = 85.  Keep 2: the tie |2| = |-2| at
    the threshold goes to index 2."""
    x = np.array([[0.1, -3.0, 2.0, -2.0, 0.5]], np.float32)
    q, sx, rs = a48.sparse_codes(x, 3)
    assert q.tolist() == [[0, -127, 85, -85, 0]] and rs.tolist() == [0]
    assert sx[0] == np.float32(3.0) / np.float32(127)
    q, _, _ = a48.sparse_codes(x, 2)
    assert q.tolist() == [[0, -127, 85, 0, 0]]
    q, _, _ = a48.sparse_codes(x, 1)
    assert q.tolist() == [[0, -127, 0, 0, 0]]


def test_sparse_codes_reduce_to_dense_and_agree_on_the_mask():
    rng = np.random.default_rng(7)
    t, k = 6, 300
    x = (rng.standard_normal((t, k)) * rng.uniform(0.01, 10, (t, 1))).astype(np.float32)
    x[2] = 0.0
    qd, sxd, rsd = oracle.act_quant(x)
    q, sx, rs = a48.sparse_codes(x, k)
    assert (q == qd).all() and (sx.view(np.uint32) == sxd.view(np.uint32)).all() and (rs == rsd).all()
    for keep in (1, 37, 150, 299):
        q, sx, rs = a48.sparse_codes(x, keep)
        mask = a48.keep_mask(x, keep)
        assert (q[mask] == qd[mask]).all() and not q[~mask].any()
        assert (sx.view(np.uint32) == sxd.view(np.uint32)).all()
        # sign symmetry: the mask depends on |x| only
        qn, _, _ = a48.sparse_codes(-x, keep)
        assert (qn == -q).all()


def test_sparse_codes_reject_whole_rows():
    """A NaN or Inf rejects its row even where it would not be kept; a row
    whose 127 / m overflows is rejected with status 2."""
    x = np.ones((4, 8), np.float32)
    x[0, 7] = np.nan
    x[1, 0] = np.inf
    x[2] = np.float32(2.0 ** -140)
    q, sx, rs = a48.sparse_codes(x, 2)
    assert rs.tolist() == [1, 1, 2, 0]
    assert not q[:3].any() and np.isnan(sx[:3]).all()
    assert q[3].tolist() == [127, 127, 0, 0, 0, 0, 0, 0]
