"""CPU oracle for the low-bit linear layer  y = s_w * s_x * (Q(W) . Q8(x)).

TEST INFRASTRUCTURE ONLY.  The tests, ``__graft_entry__.smoke()`` and the
bench's ``cpu_baseline`` leg are the only code allowed to import this package;
the GPU library and its binding never do, and the two share no code.

This module is a ctypes wrapper over ``oracle.c`` (plain scalar C, see its
header for the definitions and the pages they follow).  All functions take and
return NumPy arrays.  Format and scale-mode names come from ``workloads``.

Parity status: every function is pinned by tests/test_oracle_pins.py against
facts the pages fix (worked thresholds, add/sub/skip identities, the page's
binary packer, closed forms and invariants); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

FMT = {"ternary": 0, "binary": 1, "int4": 2}
SCALE = {"tensor": 0, "row": 1, "group": 2}
ROW_OK, ROW_NONFINITE, ROW_OVERFLOW = 0, 1, 2

_ERRS = {-1: "bad argument", -2: "accumulator range exceeded", -3: "non-finite input",
         -4: "invalid code or packed pattern"}


class OracleError(ValueError):
    def __init__(self, code: int, what: str):
        super().__init__(f"oracle {what}: {_ERRS.get(code, code)}")
        self.code = code


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < max(
            os.path.getmtime(os.path.join(_HERE, f)) for f in ("oracle.c", "oracle.h")):
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    i64, i32, p = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    pi32, pi64 = ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int64)
    lib.orc_layout.argtypes = [i32, i64, i64, pi32, pi64, pi64, pi64]
    lib.orc_n_groups.argtypes = [i32, i64, i64]; lib.orc_n_groups.restype = i64
    lib.orc_n_scales.argtypes = [i32, i64, i64, i64]; lib.orc_n_scales.restype = i64
    lib.orc_pack_scales.argtypes = [i32, i64, i64, i64, p, p]
    lib.orc_unpack_scales.argtypes = [i32, i64, i64, i64, p, p]
    lib.orc_weight_codes.argtypes = [i32, i32, i64, i32, i64, i64, p, p, p]
    lib.orc_pack.argtypes = [i32, i64, i64, p, p]
    lib.orc_unpack.argtypes = [i32, i64, i64, p, p]
    lib.orc_act_quant.argtypes = [i64, i64, p, p, p, p]; lib.orc_act_quant.restype = i64
    lib.orc_int_matmul.argtypes = [i64, i64, i64, i64, p, p, p]
    lib.orc_epilogue.argtypes = [i32, i64, i64, i64, p, p, p, p, p]
    lib.orc_linear.argtypes = [i32, i32, i64, i64, i64, p, p, i64, p, p, p, p, p]
    lib.orc_acc_bound_ok.argtypes = [i32, i64]
    lib.orc_num_threads.argtypes = []
    lib.orc_set_threads.argtypes = [i32]
    lib.orc_set_threads.restype = None
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise OracleError(rc, what)


def num_threads() -> int:
    return int(_load().orc_num_threads())


def set_threads(n: int) -> None:
    """Threads of the oracle's parallel loops from now on (timing only)."""
    _load().orc_set_threads(int(n))


def layout(fmt: str, n: int, k: int) -> dict:
    """Sizes of the tiled packed layout of an [n, k] matrix."""
    w, st, sk, nb = ctypes.c_int(), ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(_load().orc_layout(FMT[fmt], n, k, ctypes.byref(w), ctypes.byref(st), ctypes.byref(sk),
                              ctypes.byref(nb)), "layout")
    return {"wpl": w.value, "n_steps": st.value, "step_k": sk.value, "packed_bytes": nb.value}


def n_groups(scale: str, k: int, group: int) -> int:
    return int(_load().orc_n_groups(SCALE[scale], k, group))


def n_scales(scale: str, n: int, k: int, group: int) -> int:
    return int(_load().orc_n_scales(SCALE[scale], n, k, group))


def weight_codes(w: np.ndarray, fmt: str, scale: str, group: int = 0, tanh_premap: bool = False):
    """Latent fp32 W[n, k] -> (codes int8 [n, k], scales fp32 [1] | [n] | [n, G] in natural order)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, k = w.shape
    codes = np.empty((n, k), np.int8)
    if scale == "tensor":
        scales = np.empty((1,), np.float32)
    elif scale == "row":
        scales = np.empty((n,), np.float32)
    else:
        scales = np.empty((n, n_groups(scale, k, group)), np.float32)
    _check(_load().orc_weight_codes(FMT[fmt], SCALE[scale], group, int(tanh_premap), n, k,
                                    _ptr(w), _ptr(codes), _ptr(scales)), "weight_codes")
    return codes, scales


def pack(codes: np.ndarray, fmt: str) -> np.ndarray:
    """codes int8 [n, k] -> packed uint8 [packed_bytes] (tiled layout)."""
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    n, k = codes.shape
    out = np.empty((layout(fmt, n, k)["packed_bytes"],), np.uint8)
    _check(_load().orc_pack(FMT[fmt], n, k, _ptr(codes), _ptr(out)), "pack")
    return out


def unpack(packed: np.ndarray, fmt: str, n: int, k: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8).ravel()
    if packed.size != layout(fmt, n, k)["packed_bytes"]:
        raise OracleError(-1, "unpack extent")
    codes = np.empty((n, k), np.int8)
    _check(_load().orc_unpack(FMT[fmt], n, k, _ptr(packed), _ptr(codes)), "unpack")
    return codes


def pack_scales(scales: np.ndarray, scale: str, n: int, k: int, group: int = 0) -> np.ndarray:
    """Natural-order scales -> the packed artifact's order (group scales tiled)."""
    nat = np.ascontiguousarray(scales, dtype=np.float32).ravel()
    out = np.empty((n_scales(scale, n, k, group),), np.float32)
    _check(_load().orc_pack_scales(SCALE[scale], n, k, group, _ptr(nat), _ptr(out)), "pack_scales")
    return out


def unpack_scales(packed: np.ndarray, scale: str, n: int, k: int, group: int = 0) -> np.ndarray:
    pk = np.ascontiguousarray(packed, dtype=np.float32).ravel()
    G = n_groups(scale, k, group) if scale == "group" else 1
    out = np.empty(((n, G) if scale == "group" else ((n,) if scale == "row" else (1,))), np.float32)
    _check(_load().orc_unpack_scales(SCALE[scale], n, k, group, _ptr(pk), _ptr(out)), "unpack_scales")
    return out


def act_quant(x: np.ndarray):
    """x fp32 [t, k] -> (q int8 [t, k], sx fp32 [t], row_status int32 [t])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    t, k = x.shape
    q = np.empty((t, k), np.int8)
    sx = np.empty((t,), np.float32)
    st = np.empty((t,), np.int32)
    rc = _load().orc_act_quant(t, k, _ptr(x), _ptr(q), _ptr(sx), _ptr(st))
    if rc < 0:
        raise OracleError(int(rc), "act_quant")
    return q, sx, st


def int_matmul(q: np.ndarray, codes: np.ndarray, group: int = 0) -> np.ndarray:
    """acc int64 [t, n, G] = per-group sums of q[t, k] * codes[n, k]."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    t, k = q.shape
    n = codes.shape[0]
    G = (k + group - 1) // group if group > 0 else 1
    acc = np.empty((t, n, G), np.int64)
    _check(_load().orc_int_matmul(t, n, k, group, _ptr(q), _ptr(codes), _ptr(acc)), "int_matmul")
    return acc


def epilogue(acc: np.ndarray, sx: np.ndarray, scales: np.ndarray, scale: str):
    acc = np.ascontiguousarray(acc, dtype=np.int64)
    t, n, G = acc.shape
    sx = np.ascontiguousarray(sx, dtype=np.float32)
    sc = np.ascontiguousarray(scales, dtype=np.float32)
    y32 = np.empty((t, n), np.float32)
    y64 = np.empty((t, n), np.float64)
    _check(_load().orc_epilogue(SCALE[scale], t, n, G, _ptr(acc), _ptr(sx), _ptr(sc),
                                _ptr(y32), _ptr(y64)), "epilogue")
    return y32, y64


def linear(packed: np.ndarray, scales: np.ndarray, fmt: str, scale: str, group: int, n: int, k: int,
           q: np.ndarray, sx: np.ndarray):
    """Whole layer from packed bytes and packed scales: returns (y32 [t, n], y64 [t, n], acc int64 [t, n, G])."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8).ravel()
    sc = np.ascontiguousarray(scales, dtype=np.float32).ravel()
    q = np.ascontiguousarray(q, dtype=np.int8)
    sx = np.ascontiguousarray(sx, dtype=np.float32)
    t = q.shape[0]
    if q.shape[1] != k or packed.size != layout(fmt, n, k)["packed_bytes"] or sc.size != n_scales(scale, n, k, group):
        raise OracleError(-1, "linear shapes")
    G = n_groups(scale, k, group) if scale == "group" else 1
    y32 = np.empty((t, n), np.float32)
    y64 = np.empty((t, n), np.float64)
    acc = np.empty((t, n, G), np.int64)
    _check(_load().orc_linear(FMT[fmt], SCALE[scale], group, n, k, _ptr(packed), _ptr(sc),
                              t, _ptr(q), _ptr(sx), _ptr(y32), _ptr(y64), _ptr(acc)), "linear")
    return y32, y64, acc


def acc_bound_ok(fmt: str, k: int) -> bool:
    return bool(_load().orc_acc_bound_ok(FMT[fmt], k))


def quantize_and_pack(w: np.ndarray, fmt: str, scale: str, group: int = 0, tanh_premap: bool = False):
    """-> (packed bytes, packed scales, codes [n, k], natural-order scales)."""
    codes, scales = weight_codes(w, fmt, scale, group, tanh_premap)
    n, k = codes.shape
    return pack(codes, fmt), pack_scales(scales, scale, n, k, group), codes, scales
