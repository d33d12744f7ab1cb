"""CPU oracle for BitNet a4.8's hybrid activation codes - TEST INFRASTRUCTURE
ONLY (the tests, ``__graft_entry__.smoke()`` and the bench's ``cpu_baseline``
leg are its only users; the GPU library never imports it).

M8.8 "Native Binary and Ternary Transformers", 0x07B (BitNet a4.8): the
inputs of the attention and FFN projections are easy to quantise and get
4-bit codes; the intermediate states in front of the attention output and
FFN down projections are hard, so they are first sparsified and then get
8-bit codes.  The section gives no equations; what is computed here is the
plainest reading the rest of the pages supports:

* READING - the 4-bit input codes are the per-token absmax INT4 rule (the
  4-bit counterpart of 0x02C / 0x05C's INT8 rule, as for H-BitLinear):
  m = max |x| over the row, q = clip(rint(x * (7 / m)), -7, 7), s_x = m / 7,
  without the rotation (a4.8 has none; v2 added it).
* READING - "sparsifies" is a per-token magnitude threshold: each token row
  keeps its ``keep`` entries of largest |x| and sets the others to zero (the
  threshold is the keep-th largest magnitude; among equal magnitudes at the
  threshold, lower channel indices are kept first).  The kept row then gets
  the 127-based per-token INT8 codes of 0x02C / 0x05C.  The largest entry is
  always kept, so m and s_x are the dense row's and the kept entries' codes
  are the dense codes.
* A row holding NaN or Inf is rejected as a whole (zero codes, s_x = NaN,
  status 1), wherever the non-finite value sits; a row whose 127 / m (or
  7 / m) overflows is rejected with status 2.

Parity status: pinned by tests/test_a48_oracle_pins.py.
"""
from __future__ import annotations

import numpy as np

from . import act_quant
from .hadamard import act_quant4


def input_codes(x: np.ndarray):
    """The 4-bit input codes: (q int8 in [-7, 7], s_x fp32, row status)."""
    return act_quant4(np.asarray(x, np.float32))


def keep_mask(x: np.ndarray, keep: int) -> np.ndarray:
    """bool [t, k]: each row's ``keep`` entries of largest |x|, ties at the
    threshold to the lower index."""
    x = np.asarray(x, np.float32)
    t, k = x.shape
    if not 1 <= keep <= k:
        raise ValueError("keep must lie in [1, k]")
    mask = np.zeros((t, k), bool)
    idx = np.arange(k)
    for i in range(t):
        order = np.lexsort((idx, -np.abs(x[i])))      # by |x| descending, then by index
        mask[i, order[:keep]] = True
    return mask


def sparse_codes(x: np.ndarray, keep: int):
    """The sparse 8-bit intermediate codes: (q int8 in [-127, 127], s_x fp32,
    row status).  Entries outside the row's mask get code 0."""
    x = np.asarray(x, np.float32)
    t, k = x.shape
    finite = np.isfinite(x).all(axis=1)
    xs = np.where(finite[:, None], x, np.float32(0))
    kept = np.where(keep_mask(xs, keep), xs, np.float32(0))
    q, sx, rs = act_quant(kept)
    q[~finite] = 0
    sx[~finite] = np.nan
    rs[~finite] = 1
    return q, sx, rs
