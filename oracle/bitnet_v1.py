"""CPU oracle for the original BitNet BitLinear forward - TEST INFRASTRUCTURE
ONLY (the tests, ``__graft_entry__.smoke()`` and the bench's ``cpu_baseline``
leg are its only users; the GPU library never imports it).

M8.8 "Native Binary and Ternary Transformers", 0x02B-0x02E (BitNet v1):

* weights: binarised around their mean, code = +1 where w - alpha > 0 and -1
  otherwise (a tie goes to -1), alpha the mean of the scale domain; the scale
  stays the mean absolute value (0x02B);
* activations: the normalised input x_norm = SubLN(x) is coded with
  Q_b = 128: gamma = max |x_norm| over the token row (inference) or the whole
  tensor (training), code = clamp(round(x_norm * 128 / (gamma + eps)), -128,
  127), reconstruction scale gamma / 128 (0x02C, the forward of 0x02E);
* the product is the exact integer sum, rescaled by beta * gamma / 128
  (0x02D), which is the library's existing epilogue with s_x = gamma / 128.

READINGS (the pages leave these open):
* alpha is the binary64 sum of the domain's values in ascending index order,
  divided by the count and rounded once to fp32 (the reading the absmean
  scale already uses); w - alpha > 0 is decided in fp32, i.e. w > alpha.
* the activation arithmetic is fp32 in the forward's own order: d =
  fp32(gamma + fp32(eps)), then each code from fp32(fp32(x * 128) / d),
  rounded half to even; s_x = gamma / 128.
* a row whose gamma is 0 gets zero codes and s_x = 0 also when eps = 0
  (the forward states that a zero row produces zero codes and output);
* rows holding NaN or Inf are rejected (zero codes, s_x = NaN, status 1), as
  the int8 quantiser rejects them; so are rows whose max |x| * 128 overflows
  fp32 (status 2).  In per-tensor mode the tensor has one scale and one
  verdict: a non-finite value anywhere rejects every row (status 1), else a
  128 gamma that overflows does (status 2); rejected rows get zero codes and
  s_x = NaN.
* SubLN is LayerNorm without an affine map unless a gain / bias is given:
  (x - mean) / sqrt(var + eps_ln), population variance, eps_ln = 1e-5; here
  in binary64 (it feeds the quantiser through a rounding to fp32).

Parity status: pinned by tests/test_bitnet_v1_oracle_pins.py.
"""
from __future__ import annotations

import numpy as np

QB = 128
EPS = 1e-5          # the forward's default encoder epsilon
LN_EPS = 1e-5


def _domains(n: int, k: int, scale: str, group: int):
    """(row slice, column slice) of every scale domain, in the packer's order."""
    if scale == "tensor":
        return [(slice(0, n), slice(0, k))]
    span = group if scale == "group" else k
    return [(slice(r, r + 1), slice(c, min(k, c + span))) for r in range(n) for c in range(0, k, span)]


def domain_mean(values: np.ndarray) -> np.float32:
    """fp32(sum in binary64, ascending index order / count)."""
    v = np.asarray(values, np.float32).ravel().astype(np.float64)
    total = np.cumsum(v)[-1] if v.size else 0.0     # cumsum: strictly sequential
    return np.float32(total / v.size)


def centered_binary_codes(w: np.ndarray, scale: str = "tensor", group: int = 0) -> np.ndarray:
    """Centered sign codes int8 [n, k]: +1 where w > mean(domain), else -1."""
    w = np.asarray(w, np.float32)
    if not np.isfinite(w).all():
        raise ValueError("non-finite latent weight")
    n, k = w.shape
    codes = np.empty((n, k), np.int8)
    for rs, cs in _domains(n, k, scale, group):
        alpha = domain_mean(w[rs, cs])
        codes[rs, cs] = np.where(w[rs, cs] > alpha, 1, -1).astype(np.int8)
    return codes


def act_quant_v1(x: np.ndarray, per_tensor: bool = False, eps: float = EPS):
    """Q_b = 128 activation codes: returns (codes int8 [t, k] in [-128, 127],
    s_x fp32 [t] = gamma / 128, row status 0 / 1 non-finite / 2 overflow)."""
    x = np.asarray(x, np.float32)
    t, k = x.shape
    q = np.zeros((t, k), np.int8)
    sx = np.full(t, np.nan, np.float32)
    rs = np.zeros(t, np.int32)
    finite = np.isfinite(x).all(axis=1)
    with np.errstate(over="ignore", invalid="ignore"):
        amax = np.where(finite, np.abs(np.where(np.isfinite(x), x, 0)).max(axis=1), np.float32(0)).astype(np.float32)
        over = finite & ~np.isfinite(amax * np.float32(QB))
    rs[~finite] = 1
    rs[over] = 2
    if per_tensor:                                # one scale, so one verdict for every row:
        if (rs == 1).any():                       # non-finite anywhere,
            return q, sx, np.ones(t, np.int32)
        if (rs == 2).any():                       # else 128 * gamma overflowing
            return q, sx, np.full(t, 2, np.int32)
        gam = np.full(t, amax.max() if t else 0, np.float32)
    else:
        gam = amax
    e32 = np.float32(eps)
    for i in range(t):
        if rs[i]:
            continue
        if gam[i] == 0:                           # a zero row: zero codes and output (0x02E)
            sx[i] = np.float32(0)
            continue
        d = np.float32(gam[i] + e32)
        v = (x[i] * np.float32(QB)) / d           # fp32: exact * 128, then one rounded division
        q[i] = np.clip(np.rint(v), -QB, QB - 1).astype(np.int8)
        sx[i] = gam[i] / np.float32(QB)
    return q, sx, rs


def layer_norm(x: np.ndarray, eps: float = LN_EPS, gain=None, bias=None) -> np.ndarray:
    """SubLN: (x - mean) / sqrt(var + eps) per row, binary64, optional affine."""
    x = np.asarray(x, np.float64)
    mu = x.mean(axis=1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=1, keepdims=True)
    y = (x - mu) / np.sqrt(var + eps)
    if gain is not None:
        y = y * np.asarray(gain, np.float64)
    if bias is not None:
        y = y + np.asarray(bias, np.float64)
    return y
