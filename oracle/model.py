"""CPU oracle for one decode step of the 256-d ternary decoder - TEST
INFRASTRUCTURE ONLY (the tests, ``__graft_entry__.smoke()`` and the bench's
``cpu_baseline`` leg are its only users; the GPU library never imports it).

The model is the quick-start configuration of the add/sub-only inference
engine (Atomic-1Bit README, benchmark and "Quick Start" sections: 256-d, 6
layers, 4 heads, a 4096-entry vocabulary, a 128-token context, the token
embedding kept in fp32) with the projection shapes of the 256-d decode stack
(q/k/v fused [768, 256], o [256, 256], gate and up [1024, 256], down
[256, 1024], a ternary head [4096, 256]).  Its block is the LLaMA-like recipe
the b1.58 models are built on (M8.8 "Native Binary and Ternary Transformers",
the b1.58 section: RMSNorm, SwiGLU, rotary position embeddings, bias-free
linear layers), every linear layer a BitLinear: per-token absmax int8 codes of
its input times ternary codes, rescaled (same page, 0x02C-0x02D).

Arithmetic: the float steps (norm, rotation, attention, gate) are written in
binary64 from their definitions; every BitLinear takes its input rounded to
fp32 and runs the fp32 quantiser and the exact integer product of the main
oracle (``oracle.act_quant``, ``oracle.linear``), since that is where the
precision decides integers.  Readings of points the pages leave open are
marked READING.

Parity status: every function here is pinned by tests/test_oracle_pins.py
(closed forms, invariants and special cases; see each test's docstring).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List

import numpy as np

from . import act_quant, linear

# READING: the pages name RMSNorm without its epsilon; 1e-6 is the value the
# LLaMA-family recipe uses.
NORM_EPS = 1e-6
# READING: rotary embeddings with base 10000, each head's dimension i paired
# with i + head_dim / 2 ("rotate half"); the pages name RoPE only.
ROPE_BASE = 10000.0


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float = NORM_EPS) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * g over the last axis, in binary64."""
    x = np.asarray(x, np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(g, np.float64)


def rope(v: np.ndarray, pos: int, n_heads: int, base: float = ROPE_BASE) -> np.ndarray:
    """Rotate each head's pairs (i, i + hd/2) of v [n_heads * hd] by the angle
    pos * base^(-2 i / hd), i = 0 .. hd/2 - 1 (binary64)."""
    v = np.asarray(v, np.float64).reshape(n_heads, -1)
    hd = v.shape[1]
    half = hd // 2
    i = np.arange(half, dtype=np.float64)
    ang = pos * base ** (-2.0 * i / hd)
    c, s = np.cos(ang), np.sin(ang)
    a, b = v[:, :half], v[:, half:]
    out = np.empty_like(v)
    out[:, :half] = a * c - b * s
    out[:, half:] = a * s + b * c
    return out.reshape(-1)


def attend(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, n_heads: int) -> np.ndarray:
    """Causal single-token attention: q [d], caches [p + 1, d] (every cached
    position is visible).  Per head: scores q . k_j / sqrt(hd), softmax over
    j, output sum_j p_j v_j (binary64)."""
    q = np.asarray(q, np.float64).reshape(n_heads, -1)
    kc = np.asarray(k_cache, np.float64).reshape(k_cache.shape[0], n_heads, -1)
    vc = np.asarray(v_cache, np.float64).reshape(v_cache.shape[0], n_heads, -1)
    hd = q.shape[1]
    out = np.empty_like(q)
    for h in range(n_heads):
        s = kc[:, h, :] @ q[h] / np.sqrt(hd)
        e = np.exp(s - s.max())
        p = e / e.sum()
        out[h] = p @ vc[:, h, :]
    return out.reshape(-1)


def swiglu(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    """SiLU(gate) * up with SiLU(z) = z / (1 + e^-z) (binary64)."""
    g = np.asarray(gate, np.float64)
    return g / (1.0 + np.exp(-g)) * np.asarray(up, np.float64)


def bitlinear(x: np.ndarray, packed: np.ndarray, scales: np.ndarray, n: int, k: int) -> np.ndarray:
    """One BitLinear of the model (ternary codes, one fp32 scale per tensor)
    on one token: x rounded to fp32, per-token int8 codes, exact integer
    product, fp32 rescale.  Returns y [n] as fp32."""
    x32 = np.asarray(x, np.float32).reshape(1, k)
    q, sx, rs = act_quant(x32)
    if rs[0] != 0:
        raise ValueError("activation row rejected by the quantiser")
    y32, _, _ = linear(packed, scales, "ternary", "tensor", 0, n, k, q, sx)
    return y32.reshape(n).astype(np.float32)


@dataclass
class Model:
    """Weights of the decoder as the oracle sees them (host arrays)."""
    d: int
    n_layers: int
    n_heads: int
    d_ff: int
    vocab: int
    context: int
    embed: np.ndarray            # [vocab, d] fp32
    norms: np.ndarray            # [2 * n_layers + 1, d] fp32: attn_0, ffn_0, ..., final
    packed: List[np.ndarray]     # per projection, layer-major (qkv, o, gate, up, down), then the head
    scales: List[np.ndarray]

    def proj(self, layer: int, which: int):
        i = 5 * layer + which if layer < self.n_layers else 5 * self.n_layers
        return self.packed[i], self.scales[i]


PROJ_QKV, PROJ_O, PROJ_GATE, PROJ_UP, PROJ_DOWN = range(5)


def decode_step(m: Model, token: int, pos: int, k_cache: np.ndarray, v_cache: np.ndarray):
    """One decode step: the embedding row of `token` at position `pos` through
    every block (pre-norm attention and SwiGLU FFN with residual adds), the
    final norm, the head, and the greedy next token (argmax, the lowest index
    on ties).  k_cache / v_cache [n_layers, context, d] receive this position's
    rotated keys and values.  Returns (logits fp32 [vocab], next token, the
    per-layer intermediates)."""
    d, ff = m.d, m.d_ff
    x = m.embed[token].astype(np.float64)
    trace: List[Dict[str, np.ndarray]] = []
    for l in range(m.n_layers):
        t: Dict[str, np.ndarray] = {"x_in": x.copy()}
        h = rmsnorm(x, m.norms[2 * l])
        qkv = bitlinear(h, *m.proj(l, PROJ_QKV), 3 * d, d).astype(np.float64)
        q = rope(qkv[:d], pos, m.n_heads)
        k = rope(qkv[d:2 * d], pos, m.n_heads)
        v = qkv[2 * d:]
        k_cache[l, pos] = k
        v_cache[l, pos] = v
        att = attend(q, k_cache[l, :pos + 1], v_cache[l, :pos + 1], m.n_heads)
        o = bitlinear(att, *m.proj(l, PROJ_O), d, d).astype(np.float64)
        x = x + o
        h2 = rmsnorm(x, m.norms[2 * l + 1])
        gate = bitlinear(h2, *m.proj(l, PROJ_GATE), ff, d).astype(np.float64)
        up = bitlinear(h2, *m.proj(l, PROJ_UP), ff, d).astype(np.float64)
        a = swiglu(gate, up)
        dn = bitlinear(a, *m.proj(l, PROJ_DOWN), d, ff).astype(np.float64)
        x = x + dn
        t.update(h=h, qkv=qkv, q=q, k=k, attn=att, o=o, h2=h2, gate=gate, up=up, a=a, down=dn, x_out=x.copy())
        trace.append(t)
    hf = rmsnorm(x, m.norms[2 * m.n_layers])
    logits = bitlinear(hf, *m.proj(m.n_layers, 0), m.vocab, d)
    nxt = int(np.argmax(logits))
    return logits, nxt, trace
