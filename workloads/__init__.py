"""Seeded synthetic inputs for the low-bit linear layer, shared by the tests, the
bench and the oracle's callers.

This module holds shapes and random draws only: no quantisation, packing or
product arithmetic lives here, so that both the GPU path and the CPU oracle can
be fed the same bytes without sharing any of the method's code.

Every draw comes from NumPy's PCG64 seeded by
``SeedSequence([config, layer, matrix, kind])`` with kind 0 = latent weights,
1 = activations, 2 = outlier-channel choice.  Latent weights are
``0.02 * N(0, 1)`` in float32 (the std the 4-bit QAT model card reports for its
trained weights, "Weight Stability" table); activations are ``N(0, 1)`` float32.

The five workload shapes are the ones the native binary/ternary/4-bit
transformer pages train or serve:

* ``single_ternary``  - one ternary projection [768, 192] with 256 tokens.
* ``decode_stack``    - the 256-d, 6-layer ternary decoder of the add/sub-only
  inference engine's quick-start model (plus a gated FFN and a 4096 head), one
  token per call.
* ``binary_gqa``      - the 8-layer, d=192, 4x48-head / 2-KV-head INT1 model of
  the FP4-optimizer article, 32 x 256 tokens per call.
* ``ternary_4b``      - a 4B-class ternary decoder layer (K=2560, FFN 9728),
  36 layer-equivalents, group-128 scales, 1/4/16 tokens with 1 % outlier
  channels.
* ``int4_t4nt``       - the 535M-parameter 4-bit QAT model (d=1280, FFN 3584,
  20 layers), 16 x 256 prefill tokens.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Tuple

import numpy as np

# Format / scale-mode names used by every caller (the numeric codes of the C
# interface are mapped from these names by each side separately).
TERNARY, BINARY, INT4 = "ternary", "binary", "int4"
TENSOR, ROW, GROUP = "tensor", "row", "group"

WEIGHT_STD = np.float32(0.02)
KIND_W, KIND_X, KIND_OUTLIER, KIND_EMBED, KIND_NORM, KIND_TOKENS = 0, 1, 2, 3, 4, 5


@dataclass(frozen=True)
class Matrix:
    """One weight matrix of a workload: W is [n, k] (row-major, k contiguous)."""
    name: str
    n: int
    k: int
    count: int          # how many distinct copies one pass touches (layers)


@dataclass(frozen=True)
class Workload:
    index: int                      # the seed's first word
    name: str
    fmt: str                        # ternary | binary | int4
    scale: str                      # tensor | row | group
    group: int                      # columns per scale group (group mode), else 0
    tanh_premap: bool               # w -> 3 tanh(w / 3) before quantising
    layers: int
    matrices: Tuple[Matrix, ...]
    tokens: Tuple[int, ...]         # activation rows per call (one entry per T case)
    outlier_frac: float = 0.0       # fraction of channels scaled by outlier_gain
    outlier_gain: float = 10.0
    path: str = "gemv"              # the entry point the workload stresses
    notes: str = ""

    def total_weights(self) -> int:
        return sum(m.n * m.k * m.count for m in self.matrices)


def _m(name, n, k, count):
    return Matrix(name, n, k, count)


WORKLOADS: List[Workload] = [
    Workload(0, "single_ternary", TERNARY, TENSOR, 0, False, 1,
             (_m("w", 768, 192, 1),), (256,), path="both",
             notes="smallest instance; parity case for both entry points"),
    Workload(1, "decode_stack", TERNARY, TENSOR, 0, False, 6,
             (_m("qkv", 768, 256, 6), _m("o", 256, 256, 6), _m("up", 1024, 256, 6),
              _m("gate", 1024, 256, 6), _m("down", 256, 1024, 6), _m("head", 4096, 256, 1)),
             (1,), path="gemv",
             notes="batch-1 decode over a 256-d 6-layer stack; every matrix cache-resident"),
    Workload(2, "binary_gqa", BINARY, ROW, 0, False, 8,
             (_m("q", 192, 192, 8), _m("k", 96, 192, 8), _m("v", 96, 192, 8), _m("o", 192, 192, 8),
              _m("up", 768, 192, 8), _m("gate", 768, 192, 8), _m("down", 192, 768, 8)),
             (8192,), path="gemm",
             notes="binary weights, per-row absmean scale, 8192-token batched GEMM"),
    Workload(3, "ternary_4b", TERNARY, GROUP, 128, False, 36,
             (_m("attn0", 2560, 2560, 36), _m("attn1", 2560, 2560, 36), _m("attn2", 2560, 2560, 36),
              _m("attn3", 2560, 2560, 36), _m("gate", 9728, 2560, 36), _m("up", 9728, 2560, 36),
              _m("down", 2560, 9728, 36)),
             (1, 4, 16), outlier_frac=0.01, path="gemv",
             notes="HBM-bound decode GEMV; ~1.03 GB of packed codes + scales per pass"),
    Workload(4, "int4_t4nt", INT4, ROW, 0, True, 20,
             (_m("qkv", 3840, 1280, 20), _m("o", 1280, 1280, 20), _m("up", 3584, 1280, 20),
              _m("gate", 3584, 1280, 20), _m("down", 1280, 3584, 20)),
             (4096,), path="gemm",
             notes="int4 levels -7..+7 with tanh soft clipping; 4096-token prefill GEMM"),
]

BY_NAME = {w.name: w for w in WORKLOADS}


def _rng(workload: int, layer: int, matrix: int, kind: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([workload, layer, matrix, kind])))


def latent_weights(workload: int, layer: int, matrix: int, n: int, k: int) -> np.ndarray:
    """Latent fp32 weights W[n, k] = 0.02 * N(0, 1)."""
    w = _rng(workload, layer, matrix, KIND_W).standard_normal((n, k), dtype=np.float32)
    w *= WEIGHT_STD
    return w


def activations(workload: int, layer: int, matrix: int, t: int, k: int,
                outlier_frac: float = 0.0, outlier_gain: float = 10.0) -> np.ndarray:
    """Activations x[t, k] = N(0, 1) fp32; optionally ceil(frac * k) channels
    (a seeded choice, the same columns for every token) multiplied by ``gain``."""
    x = _rng(workload, layer, matrix, KIND_X).standard_normal((t, k), dtype=np.float32)
    if outlier_frac > 0.0:
        n_out = int(math.ceil(outlier_frac * k))
        cols = _rng(workload, layer, matrix, KIND_OUTLIER).choice(k, size=n_out, replace=False)
        x[:, np.sort(cols)] *= np.float32(outlier_gain)
    return x


def workload_activations(wl: Workload, layer: int, matrix: int, t: int, k: int) -> np.ndarray:
    return activations(wl.index, layer, matrix, t, k, wl.outlier_frac, wl.outlier_gain)


def random_case(seed: int, n: int, k: int, t: int, scale: float = 0.02) -> Tuple[np.ndarray, np.ndarray]:
    """Weights and activations for ad-hoc shapes (ragged-tail and edge tests)."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([1000, seed])))
    w = g.standard_normal((n, k), dtype=np.float32) * np.float32(scale)
    x = g.standard_normal((t, k), dtype=np.float32)
    return w, x


# ---------------------------------------------------------------- decode model
# The 256-d decoder the decode-stack matrices belong to, as a whole model:
# the add/sub-only engine's quick-start configuration (256-d, 6 layers, 4
# heads, 4096-entry vocabulary, 128-token context) with the stack's gated FFN.
DECODE_MODEL = dict(d=256, layers=6, heads=4, d_ff=1024, vocab=4096, context=128)


def decode_model_embedding(vocab: int, d: int) -> np.ndarray:
    """Token embedding table [vocab, d] = N(0, 1) fp32 (kept in fp32, as the
    engine's README keeps it)."""
    return _rng(1, 0, 0, KIND_EMBED).standard_normal((vocab, d), dtype=np.float32)


def decode_model_norms(layers: int, d: int) -> np.ndarray:
    """RMSNorm gains [2 * layers + 1, d] = 1 + 0.1 N(0, 1) fp32 (attention and
    FFN norm of each layer, then the final norm)."""
    g = _rng(1, 0, 0, KIND_NORM).standard_normal((2 * layers + 1, d), dtype=np.float32)
    return (np.float32(1.0) + np.float32(0.1) * g).astype(np.float32)


def decode_model_tokens(n: int, vocab: int, seed: int = 0) -> np.ndarray:
    """n seeded token ids in [0, vocab)."""
    return _rng(1, seed, 0, KIND_TOKENS).integers(0, vocab, size=n, dtype=np.int64).astype(np.int32)
