"""CPU oracle for OneBit's W1A16 linear layer - TEST INFRASTRUCTURE ONLY (the
tests, ``__graft_entry__.smoke()`` and the bench's ``cpu_baseline`` leg are
its only users; the GPU library never imports it).

M8.8 "Native Binary and Ternary Transformers", 0x06A (OneBit): a trained FP
matrix is replaced by a sign matrix S in {-1, +1}^[N, K], an FP16 vector g
over the input dimension and an FP16 vector h over the output dimension, and
a LayerNorm follows the binary projection:

    y = LayerNorm(((x * g) S^T) * h)           x: [T, K], activations in FP16

The section's forward multiplies x by g first, contracts with the signs, then
scales by h and normalises; the sign is +1 at either signed zero (0x06D's
forward), which is the binary packer's rule.

READINGS (the pages leave these open):
* x, g and h are FP16 (W1A16); x * g is rounded to FP16 (the elementwise
  product of two FP16 tensors), the contraction is exact here (binary64 of
  the FP16 operands; the kernel accumulates in fp32), the output is not
  rounded back to FP16: the projection and the layer return fp32 / binary64;
* the LayerNorm after it normalises each token's N outputs, population
  variance, eps 1e-5, with an optional affine map (oracle.bitnet_v1's).

Parity status: pinned by tests/test_onebit_oracle_pins.py.
"""
from __future__ import annotations

import numpy as np

from .bitnet_v1 import layer_norm


def signs(w: np.ndarray) -> np.ndarray:
    """The sign matrix of latent weights: +1 where w >= 0 (either zero), else -1."""
    w = np.asarray(w, np.float32)
    return np.where(w >= 0, 1, -1).astype(np.int8)


def scaled_input(x16: np.ndarray, g16: np.ndarray) -> np.ndarray:
    """x * g as FP16 (one rounding of the exact product)."""
    return (np.asarray(x16, np.float16).astype(np.float32) * np.asarray(g16, np.float16).astype(np.float32)).astype(
        np.float16)


def projection(x16: np.ndarray, g16: np.ndarray, s: np.ndarray, h16: np.ndarray) -> np.ndarray:
    """((x * g) S^T) * h in binary64: [T, N]."""
    xg = scaled_input(x16, g16).astype(np.float64)
    return (xg @ np.asarray(s, np.float64).T) * np.asarray(h16, np.float16).astype(np.float64)[None, :]


def onebit_linear(x16, g16, s, h16, ln_eps: float = 1e-5, gain=None, bias=None) -> np.ndarray:
    """The whole layer: LayerNorm of the projection over the output dimension."""
    return layer_norm(projection(x16, g16, s, h16), ln_eps, gain, bias)
