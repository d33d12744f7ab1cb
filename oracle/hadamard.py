"""CPU oracle for the rotated 4-bit activation quantiser of H-BitLinear - TEST
INFRASTRUCTURE ONLY (the tests, ``__graft_entry__.smoke()`` and the bench's
``cpu_baseline`` leg are its only users; the GPU library never imports it).

M8.8 "Native Binary and Ternary Transformers", 0x07C (BitNet v2): before
activation quantisation, an online Hadamard transform, computed fast in
O(K log K), spreads channel outliers, and the activations are then quantised
to INT4.  The section's equation did not survive; what is computed here is the
plainest reading the rest supports:

* READING - the transform is the orthonormal Walsh-Hadamard transform
  (Sylvester order), applied block-diagonally over consecutive blocks of B
  channels, B the largest power of two dividing K (up to 2048): a full
  transform when K is a power of two, and the O(K log K) fast form either way.
* READING - INT4 codes are the 4-bit counterpart of the per-token absmax rule
  the page states for INT8 (0x02C, 0x05C): m = max |x'| over the row,
  r = 7 / m, q = clip(rint(x' r), -7, 7), s_x = m / 7; a row with a non-finite
  value, or whose 7 / m overflows, is rejected.
* The precision that decides the codes is fp32 (the quantiser's, as for INT8):
  the transform runs as fp32 butterflies, stage by stage (half-width h = 1,
  2, 4, ..., B / 2; each pair (a, b) -> (a + b, a - b)), then a multiply by
  fp32(1 / sqrt(B)).  The pins check that against the dense binary64
  definition.

Parity status: pinned by tests/test_hadamard_oracle_pins.py.
"""
from __future__ import annotations

import numpy as np

QMAX4 = 7


def block_size(k: int) -> int:
    """The largest power of two dividing k, at most 2048 (0 when below 64:
    the transform is defined here for blocks of 64 and more)."""
    b = k & -k
    b = min(b, 2048)
    return b if b >= 64 else 0


def fwht_blocks(x: np.ndarray, b: int) -> np.ndarray:
    """Orthonormal Walsh-Hadamard transform of each length-b block of the
    rows of x (fp32, butterflies stage by stage, then * fp32(1/sqrt(b)))."""
    x = np.asarray(x, np.float32)
    t, k = x.shape
    assert k % b == 0 and b & (b - 1) == 0
    v = x.reshape(t, k // b, b).copy()
    h = 1
    with np.errstate(over="ignore", invalid="ignore"):   # Inf / NaN rows are rejected later
        while h < b:
            w = v.reshape(t, k // b, b // (2 * h), 2, h)
            a = w[:, :, :, 0, :].copy()
            c = w[:, :, :, 1, :].copy()
            w[:, :, :, 0, :] = a + c
            w[:, :, :, 1, :] = a - c
            h *= 2
        scale = np.float32(1.0 / np.sqrt(np.float64(b)))
        return (v * scale).reshape(t, k).astype(np.float32)


def act_quant4(xr: np.ndarray):
    """Per-token absmax INT4 codes of already-rotated rows (fp32): returns
    (codes int8 in [-7, 7], s_x fp32, row status 0 ok / 1 non-finite /
    2 overflow).  Rejected rows get zero codes and s_x = NaN."""
    xr = np.asarray(xr, np.float32)
    t, k = xr.shape
    q = np.zeros((t, k), np.int8)
    sx = np.zeros(t, np.float32)
    rs = np.zeros(t, np.int32)
    for i in range(t):
        row = xr[i]
        if not np.isfinite(row).all():
            rs[i], sx[i] = 1, np.nan
            continue
        m = np.float32(np.abs(row).max()) if k else np.float32(0)
        if m == 0:
            continue
        with np.errstate(over="ignore"):
            r = np.float32(QMAX4) / m
        if not np.isfinite(r):
            rs[i], sx[i] = 2, np.nan
            continue
        q[i] = np.clip(np.rint(row * r), -QMAX4, QMAX4).astype(np.int8)
        sx[i] = m / np.float32(QMAX4)
    return q, sx, rs


def rotated_act_quant4(x: np.ndarray):
    """H-BitLinear's activation quantiser: block Hadamard, then INT4 codes."""
    x = np.asarray(x, np.float32)
    b = block_size(x.shape[1])
    if b == 0:
        raise ValueError("k must be a multiple of 64")
    return act_quant4(fwht_blocks(x, b))
