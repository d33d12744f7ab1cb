"""Python binding of liblowbit.so, the MI355X low-bit linear layer.

Argument marshalling only: every step (packing, activation quantisation, the
integer products and their epilogues) runs in the native library.  The
functions keep the C names of include/lowbit.h.  Device buffers are torch
tensors on the GPU (the library reads their data pointers and launches on
torch's current stream); host buffers are NumPy arrays.  The library
allocates nothing, so callers pass every output buffer.

If the shared library has not been built this module raises ImportError: there
is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblowbit.so")

TERNARY2, BINARY1, INT4 = 0, 1, 2
SCALE_TENSOR, SCALE_ROW, SCALE_GROUP = 0, 1, 2
FLAG_TANH3 = 1
FLAG_CENTERED = 2
ACT_NONFINITE, ACT_OVERFLOW = 1, 2
FORMATS = {"ternary": TERNARY2, "binary": BINARY1, "int4": INT4}
SCALES = {"tensor": SCALE_TENSOR, "row": SCALE_ROW, "group": SCALE_GROUP}
STATUS = {0: "LOWBIT_OK", 1: "LOWBIT_E_ARG", 2: "LOWBIT_E_RANGE", 3: "LOWBIT_E_NONFINITE",
          4: "LOWBIT_E_FORMAT", 5: "LOWBIT_E_HIP"}

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python -m bit_weight_linear_bitlinear_amd.build` "
                      "(or __graft_entry__.build()) first")

# torch's wheel ships its own HIP runtime.  Importing torch first makes the
# library bind to that same runtime (the dynamic linker reuses the loaded
# libamdhip64.so.7), so device pointers and streams from torch tensors are
# valid in our launches; loading the library first would put a second HIP
# runtime in the process.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)


class lowbit_desc(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("scale", ctypes.c_int32), ("n", ctypes.c_int32),
                ("k", ctypes.c_int32), ("group", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("wpl", ctypes.c_int32), ("step_k", ctypes.c_int32), ("n_steps", ctypes.c_int64),
                ("packed_bytes", ctypes.c_int64), ("n_groups", ctypes.c_int64), ("n_scales", ctypes.c_int64)]

    def __repr__(self):
        return (f"lowbit_desc(format={self.format}, scale={self.scale}, n={self.n}, k={self.k}, "
                f"group={self.group}, flags={self.flags}, wpl={self.wpl}, step_k={self.step_k}, "
                f"n_steps={self.n_steps}, "
                f"packed_bytes={self.packed_bytes}, n_groups={self.n_groups}, n_scales={self.n_scales})")


_P = ctypes.c_void_p
_D = ctypes.POINTER(lowbit_desc)
_i32 = ctypes.c_int32
_lib.lowbit_describe.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, _D]
_lib.lowbit_pack.argtypes = [_D, _P, _P, _P]
_lib.lowbit_act_quant.argtypes = [_P, _i32, _i32, _P, _P, _P, _P]
_lib.lowbit_act_quant_h4.argtypes = [_P, _i32, _i32, _P, _P, _P, _P]
_lib.lowbit_act_quant_h4.restype = _i32
_lib.lowbit_act_quant_a4.argtypes = [_P, _i32, _i32, _P, _P, _P, _P]
_lib.lowbit_act_quant_a4.restype = _i32
_lib.lowbit_act_quant_sparse8.argtypes = [_P, _i32, _i32, _i32, _P, _P, _P, _P]
_lib.lowbit_act_quant_sparse8.restype = _i32
_lib.lowbit_act_quant_v1.argtypes = [_P, _i32, _i32, ctypes.c_float, _i32, _P, _P, _P, _P, _P]
_lib.lowbit_act_quant_v1.restype = _i32
_lib.lowbit_layernorm.argtypes = [_P, _i32, _i32, ctypes.c_float, _P, _P, _P, _P]
_lib.lowbit_layernorm.restype = _i32
_lib.lowbit_onebit_linear.argtypes = [_D, _P, _P, _P, _P, _i32, _P, _P]
_lib.lowbit_onebit_linear.restype = _i32
_lib.lowbit_linear.argtypes = [_D, _P, _P, _P, _P, _i32, _P, _P, _P]
_lib.lowbit_linear_batched.argtypes = [_D, _P, _P, _P, _P, _i32, _P, _P, _P]
_PP = ctypes.POINTER(ctypes.c_void_p)
_lib.lowbit_linear_grouped.argtypes = [_i32, _D, _PP, _PP, _PP, _PP, _i32, _PP, _PP, _P]
_lib.lowbit_linear_grouped.restype = _i32
_lib.lowbit_linear_batched_grouped.argtypes = [_i32, _D, _PP, _PP, _PP, _PP, _i32, _PP, _PP, _P]
_lib.lowbit_linear_batched_grouped.restype = _i32
_lib.lowbit_linear_fused.argtypes = [_D, _P, _P, _P, _i32, _P, _P, _P, _P, _P]
_lib.lowbit_linear_fused.restype = _i32
_lib.lowbit_linear_grouped_fused.argtypes = [_i32, _D, _PP, _PP, _PP, _PP, _PP, _i32, _PP, _P, _P]
_lib.lowbit_linear_grouped_fused.restype = _i32


class lowbit_model(ctypes.Structure):
    """Mirror of the C struct lowbit_model (one decode step's model)."""
    _fields_ = [("d_model", ctypes.c_int32), ("n_layers", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("d_ff", ctypes.c_int32), ("vocab", ctypes.c_int32), ("context", ctypes.c_int32),
                ("norm_eps", ctypes.c_float), ("rope_base", ctypes.c_float), ("proj", lowbit_desc * 6),
                ("embed", _P), ("norms", _P), ("packed", _PP), ("scales", _PP), ("k_cache", _P),
                ("v_cache", _P), ("work", _P)]


_M = ctypes.POINTER(lowbit_model)
_lib.lowbit_model_work_bytes.argtypes = [_M]
_lib.lowbit_model_work_bytes.restype = ctypes.c_int64
_lib.lowbit_model_trace_floats.argtypes = [_M]
_lib.lowbit_model_trace_floats.restype = ctypes.c_int64
_lib.lowbit_decode_step.argtypes = [_M, _P, _P, _P, _P, _P]
_lib.lowbit_decode_step.restype = _i32
_lib.lowbit_decode_step_noalloc.argtypes = [_M, _P, _P, _P, _P, _P]
_lib.lowbit_decode_step_noalloc.restype = _i32
NOALLOC_WORK_BYTES = 1 << 20
_lib.lowbit_rmsnorm.argtypes = [_P, _P, _P, _P, _i32, _i32, ctypes.c_float, _P, _P]
_lib.lowbit_rmsnorm.restype = _i32
_lib.lowbit_rope_attention.argtypes = [_P, _i32, _i32, _i32, ctypes.c_float, _P, _P, _P, _P]
_lib.lowbit_rope_attention.restype = _i32
_lib.lowbit_swiglu.argtypes = [_P, _P, ctypes.c_int64, _P, _P]
_lib.lowbit_swiglu.restype = _i32
_lib.lowbit_calib_read.argtypes = [_P, ctypes.c_int64, _P, _P]
_lib.lowbit_calib_read.restype = _i32
_lib.lowbit_calib_mfma_i8.argtypes = [_i32, _P, _P]
_lib.lowbit_calib_mfma_i8.restype = _i32
_lib.lowbit_calib_mfma_i8_ops.argtypes = [_i32]
_lib.lowbit_calib_mfma_i8_ops.restype = ctypes.c_int64
_lib.lowbit_max_k.argtypes = [_i32]
_lib.lowbit_max_k.restype = _i32
_lib.lowbit_status_string.argtypes = [_i32]
_lib.lowbit_status_string.restype = ctypes.c_char_p
_lib.lowbit_abi_version.restype = _i32
_lib.lowbit_last_hip_error.restype = ctypes.c_char_p
for _f in ("lowbit_describe", "lowbit_pack", "lowbit_act_quant", "lowbit_linear", "lowbit_linear_batched"):
    getattr(_lib, _f).restype = _i32

EXPORTS = ("lowbit_describe", "lowbit_pack", "lowbit_act_quant", "lowbit_act_quant_h4", "lowbit_act_quant_a4",
           "lowbit_act_quant_sparse8", "lowbit_act_quant_v1",
           "lowbit_layernorm", "lowbit_onebit_linear", "lowbit_linear",
           "lowbit_linear_batched",
           "lowbit_linear_grouped", "lowbit_linear_batched_grouped", "lowbit_linear_fused",
           "lowbit_linear_grouped_fused",
           "lowbit_model_work_bytes", "lowbit_model_trace_floats", "lowbit_decode_step", "lowbit_decode_step_noalloc",
           "lowbit_rmsnorm", "lowbit_rope_attention", "lowbit_swiglu",
           "lowbit_calib_read", "lowbit_calib_mfma_i8", "lowbit_calib_mfma_i8_ops",
           "lowbit_max_k", "lowbit_status_string", "lowbit_abi_version", "lowbit_last_hip_error")

# projection slots (lowbit_model.proj and the per-layer weight lists)
PROJ_QKV, PROJ_O, PROJ_GATE, PROJ_UP, PROJ_DOWN, PROJ_HEAD = range(6)
STEP_POSITION, STEP_TOKEN = 1, 2


class LowbitError(RuntimeError):
    def __init__(self, status: int, call: str):
        msg = _lib.lowbit_status_string(status).decode()
        if status == 5:
            msg += ": " + _lib.lowbit_last_hip_error().decode()
        super().__init__(f"{call}: {STATUS.get(status, status)} ({msg})")
        self.status = status


def _check(status: int, call: str) -> None:
    if status != 0:
        raise LowbitError(status, call)


# element types the C ABI reads or writes behind each argument name
_F32, _I8, _U8, _I32, _F16 = "float32", "int8", "uint8", "int32", "float16"


def _types(**args):
    """Element types, checked for every argument before any other check:
    name=(tensor or list of tensors or None, dtype name or tuple of names)."""
    for name, (t, dtype) in args.items():
        allowed = (dtype,) if isinstance(dtype, str) else dtype
        for v in (t if isinstance(t, (list, tuple)) else (t,)):
            if v is not None and str(v.dtype).replace("torch.", "") not in allowed:
                raise ValueError(f"{name}: expected dtype {' or '.join(allowed)}, got {v.dtype}")


def _dev(t, name, nbytes=None):
    """Data pointer of a contiguous device tensor holding >= nbytes (None -> NULL)."""
    if t is None:
        return None
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous GPU tensor")
    if nbytes is not None and t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name}: buffer holds {t.numel() * t.element_size()} bytes, needs {nbytes}")
    return ctypes.c_void_p(t.data_ptr())


def _host(a: np.ndarray, name, dtype, count=None):
    if not isinstance(a, np.ndarray) or a.dtype != dtype or not a.flags.c_contiguous:
        raise ValueError(f"{name}: expected a C-contiguous numpy {np.dtype(dtype).name} array")
    if count is not None and a.size < count:
        raise ValueError(f"{name}: array holds {a.size} elements, needs {count}")
    return a.ctypes.data_as(ctypes.c_void_p)


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def lowbit_describe(format: int, scale: int, n: int, k: int, group: int = 0, flags: int = 0) -> lowbit_desc:
    d = lowbit_desc()
    _check(_lib.lowbit_describe(format, scale, n, k, group, flags, ctypes.byref(d)), "lowbit_describe")
    return d


def lowbit_pack(d: lowbit_desc, w: np.ndarray, packed: np.ndarray, scales: np.ndarray) -> None:
    """Host: latent fp32 w[n, k] -> packed uint8[packed_bytes], scales fp32[n_scales]."""
    _check(_lib.lowbit_pack(ctypes.byref(d), _host(w, "w", np.float32, d.n * d.k),
                            _host(packed, "packed", np.uint8, d.packed_bytes),
                            _host(scales, "scales", np.float32, d.n_scales)), "lowbit_pack")


def lowbit_act_quant(x, q, sx, status=None, stream=None) -> None:
    """Device: x fp32[t, k] -> q int8[t, k], sx fp32[t]; status int32[1] or None."""
    _types(x=(x, _F32), q=(q, _I8), sx=(sx, _F32), status=(status, _I32))
    t, k = x.shape
    _check(_lib.lowbit_act_quant(_dev(x, "x", 4 * t * k), t, k, _dev(q, "q", t * k),
                                 _dev(sx, "sx", 4 * t), _dev(status, "status", 4), _stream(stream)),
           "lowbit_act_quant")


def lowbit_act_quant_h4(x, q, sx, status=None, stream=None) -> None:
    """Device: x fp32[t, k] -> block-Hadamard-rotated INT4 codes q int8[t, k]
    (in [-7, 7]) and sx fp32[t]; status int32[1] or None."""
    _types(x=(x, _F32), q=(q, _I8), sx=(sx, _F32), status=(status, _I32))
    t, k = x.shape
    _check(_lib.lowbit_act_quant_h4(_dev(x, "x", 4 * t * k), t, k, _dev(q, "q", t * k),
                                    _dev(sx, "sx", 4 * t), _dev(status, "status", 4), _stream(stream)),
           "lowbit_act_quant_h4")


def lowbit_act_quant_a4(x, q, sx, status=None, stream=None) -> None:
    """Device: x fp32[t, k] -> per-token INT4 codes q int8[t, k] (in [-7, 7])
    and sx fp32[t] = max|x| / 7; status int32[1] or None."""
    _types(x=(x, _F32), q=(q, _I8), sx=(sx, _F32), status=(status, _I32))
    t, k = x.shape
    _check(_lib.lowbit_act_quant_a4(_dev(x, "x", 4 * t * k), t, k, _dev(q, "q", t * k),
                                    _dev(sx, "sx", 4 * t), _dev(status, "status", 4), _stream(stream)),
           "lowbit_act_quant_a4")


def lowbit_act_quant_sparse8(x, q, sx, keep, status=None, stream=None) -> None:
    """Device: each row of x fp32[t, k] keeps its `keep` largest |x| (ties to
    the lower channel) with per-token INT8 codes, the rest code 0 -> q
    int8[t, k], sx fp32[t] = max|x| / 127; status int32[1] or None."""
    _types(x=(x, _F32), q=(q, _I8), sx=(sx, _F32), status=(status, _I32))
    t, k = x.shape
    _check(_lib.lowbit_act_quant_sparse8(_dev(x, "x", 4 * t * k), t, k, int(keep), _dev(q, "q", t * k),
                                         _dev(sx, "sx", 4 * t), _dev(status, "status", 4),
                                         _stream(stream)),
           "lowbit_act_quant_sparse8")


def lowbit_act_quant_v1(x, q, sx, eps=1e-5, per_tensor=False, status=None, work=None, stream=None) -> None:
    """Device: the original BitNet's Q_b = 128 codes of x fp32[t, k] -> q
    int8[t, k] in [-128, 127], sx fp32[t] = gamma / 128; per_tensor needs
    work, a device uint32[2] (or int32[2]) workspace."""
    _types(x=(x, _F32), q=(q, _I8), sx=(sx, _F32), status=(status, _I32), work=(work, (_I32, "uint32")))
    t, k = x.shape
    _check(_lib.lowbit_act_quant_v1(_dev(x, "x", 4 * t * k), t, k, float(eps), int(bool(per_tensor)),
                                    _dev(q, "q", t * k), _dev(sx, "sx", 4 * t),
                                    _dev(status, "status", 4), _dev(work, "work", 8),
                                    _stream(stream)), "lowbit_act_quant_v1")


def lowbit_layernorm(x, out, eps=1e-5, gain=None, bias=None, stream=None) -> None:
    """Device: out = LayerNorm(x) per row (fp32), optional gain / bias [d]."""
    _types(x=(x, _F32), out=(out, _F32), gain=(gain, _F32), bias=(bias, _F32))
    t, d = x.shape
    _check(_lib.lowbit_layernorm(_dev(x, "x", 4 * t * d), t, d, float(eps), _dev(gain, "gain", 4 * d),
                                 _dev(bias, "bias", 4 * d), _dev(out, "out", 4 * t * d), _stream(stream)),
           "lowbit_layernorm")


def lowbit_onebit_linear(d: lowbit_desc, packed, g, h, x, y, stream=None) -> None:
    """Device: OneBit's projection y fp32[t, n] = h * (fp16(x * g) . S^T) from
    x fp16[t, k], g fp16[k], h fp16[n] and binary packed signs."""
    _types(packed=(packed, _U8), g=(g, _F16), h=(h, _F16), x=(x, _F16), y=(y, _F32))
    t = x.shape[0]
    if x.dim() != 2 or x.shape[1] != d.k:
        raise ValueError(f"onebit: x: expected [t, {d.k}], got {tuple(x.shape)}")
    _check(_lib.lowbit_onebit_linear(ctypes.byref(d), _dev(packed, "packed", d.packed_bytes),
                                     _dev(g, "g", 2 * d.k), _dev(h, "h", 2 * d.n),
                                     _dev(x, "x", 2 * t * d.k), t, _dev(y, "y", 4 * t * d.n),
                                     _stream(stream)), "lowbit_onebit_linear")


def _linear_ptrs(d, packed, scales, q, sx, y, acc):
    _types(packed=(packed, _U8), scales=(scales, _F32), q=(q, _I8), sx=(sx, _F32), y=(y, _F32), acc=(acc, _I32))
    t = q.shape[0]
    if q.dim() != 2 or q.shape[1] != d.k:
        raise ValueError(f"q: expected [t, {d.k}], got {tuple(q.shape)}")
    return (_dev(packed, "packed", d.packed_bytes), _dev(scales, "scales", 4 * d.n_scales),
            _dev(q, "q", t * d.k), _dev(sx, "sx", 4 * t), t, _dev(y, "y", 4 * t * d.n),
            _dev(acc, "acc", 4 * t * d.n * d.n_groups))


def lowbit_linear(d: lowbit_desc, packed, scales, q, sx, y, acc=None, stream=None) -> None:
    """Device GEMV: y fp32[t, n] (and acc int32[t, n, n_groups] if given)."""
    _check(_lib.lowbit_linear(ctypes.byref(d), *_linear_ptrs(d, packed, scales, q, sx, y, acc), _stream(stream)),
           "lowbit_linear")


def lowbit_linear_batched(d: lowbit_desc, packed, scales, q, sx, y, acc=None, stream=None) -> None:
    """Device GEMM on the matrix cores: same contract as lowbit_linear."""
    _check(_lib.lowbit_linear_batched(ctypes.byref(d), *_linear_ptrs(d, packed, scales, q, sx, y, acc),
                                      _stream(stream)), "lowbit_linear_batched")


class GroupedCall:
    """Marshalled arguments of one lowbit_linear_grouped call (the pointer
    arrays are built once, so replaying the call costs no Python work beyond
    the foreign call itself); batched=True marshals
    lowbit_linear_batched_grouped (the prefill GEMMs) instead."""

    def __init__(self, descs, packed, scales, q, sx, y, acc=None, batched=False):
        self.batched = batched
        n = len(descs)
        if not (n == len(packed) == len(scales) == len(q) == len(sx) == len(y)) or n < 1:
            raise ValueError("lowbit_linear_grouped: argument lists differ in length")
        t = q[0].shape[0]
        arr = lambda ptrs: (ctypes.c_void_p * n)(*[p.value if p is not None else None for p in ptrs])
        cols = [_linear_ptrs(d, pk, sc, qq, ss, yy, aa) for d, pk, sc, qq, ss, yy, aa in
                zip(descs, packed, scales, q, sx, y, acc if acc is not None else [None] * n)]
        if any(c[4] != t for c in cols):
            raise ValueError("lowbit_linear_grouped: every q must have the same token count")
        self.count = n
        self.t = t
        self.descs = (lowbit_desc * n)(*descs)
        self.packed = arr([c[0] for c in cols])
        self.scales = arr([c[1] for c in cols])
        self.q = arr([c[2] for c in cols])
        self.sx = arr([c[3] for c in cols])
        self.y = arr([c[5] for c in cols])
        self.acc = arr([c[6] for c in cols]) if acc is not None else None
        self._keep = (packed, scales, q, sx, y, acc)    # the tensors must outlive the call

    def __call__(self, stream=None):
        fn = "lowbit_linear_batched_grouped" if self.batched else "lowbit_linear_grouped"
        _check(getattr(_lib, fn)(self.count, self.descs, self.packed, self.scales, self.q, self.sx,
                                 self.t, self.y, self.acc, _stream(stream)), fn)


def lowbit_linear_batched_grouped(descs, packed, scales, q, sx, y, acc=None, stream=None) -> None:
    """Device: several independent prefill GEMMs of equal k and t, at most 64 per launch."""
    GroupedCall(descs, packed, scales, q, sx, y, acc, batched=True)(stream)


def lowbit_linear_grouped(descs, packed, scales, q, sx, y, acc=None, stream=None) -> None:
    """Device: several independent GEMVs of equal k in one launch."""
    GroupedCall(descs, packed, scales, q, sx, y, acc)(stream)


def _fused_ptrs(d, packed, scales, x, q, sx, y):
    _types(packed=(packed, _U8), scales=(scales, _F32), x=(x, _F32), q=(q, _I8), sx=(sx, _F32), y=(y, _F32))
    t = x.shape[0]
    if x.dim() != 2 or x.shape[1] != d.k or tuple(q.shape) != (t, d.k):
        raise ValueError(f"x, q: expected [t, {d.k}], got {tuple(x.shape)}, {tuple(q.shape)}")
    return (_dev(packed, "packed", d.packed_bytes), _dev(scales, "scales", 4 * d.n_scales),
            _dev(x, "x", 4 * t * d.k), t, _dev(q, "q", t * d.k), _dev(sx, "sx", 4 * t),
            _dev(y, "y", 4 * t * d.n))


def lowbit_linear_fused(d: lowbit_desc, packed, scales, x, q, sx, y, status=None, stream=None) -> None:
    """Device GEMV from fp32 x: the activation quantiser runs inside the product;
    q int8[t, k] and sx fp32[t] receive the codes and scales as by-products."""
    _types(status=(status, _I32))
    _check(_lib.lowbit_linear_fused(ctypes.byref(d), *_fused_ptrs(d, packed, scales, x, q, sx, y),
                                    _dev(status, "status", 4), _stream(stream)), "lowbit_linear_fused")


class GroupedFusedCall:
    """Marshalled arguments of one lowbit_linear_grouped_fused call."""

    def __init__(self, descs, packed, scales, x, q, sx, y, status=None):
        _types(status=(status, _I32))
        n = len(descs)
        if not (n == len(packed) == len(scales) == len(x) == len(q) == len(sx) == len(y)) or n < 1:
            raise ValueError("lowbit_linear_grouped_fused: argument lists differ in length")
        cols = [_fused_ptrs(d, pk, sc, xx, qq, ss, yy) for d, pk, sc, xx, qq, ss, yy in
                zip(descs, packed, scales, x, q, sx, y)]
        t = cols[0][3]
        if any(c[3] != t for c in cols):
            raise ValueError("lowbit_linear_grouped_fused: every x must have the same token count")
        arr = lambda ptrs: (ctypes.c_void_p * n)(*[p.value for p in ptrs])
        self.count, self.t = n, t
        self.descs = (lowbit_desc * n)(*descs)
        self.packed = arr([c[0] for c in cols])
        self.scales = arr([c[1] for c in cols])
        self.x = arr([c[2] for c in cols])
        self.q = arr([c[4] for c in cols])
        self.sx = arr([c[5] for c in cols])
        self.y = arr([c[6] for c in cols])
        self.status = _dev(status, "status", 4)
        self._keep = (packed, scales, x, q, sx, y, status)

    def __call__(self, stream=None):
        _check(_lib.lowbit_linear_grouped_fused(self.count, self.descs, self.packed, self.scales, self.x, self.q,
                                                self.sx, self.t, self.y, self.status, _stream(stream)),
               "lowbit_linear_grouped_fused")


def lowbit_linear_grouped_fused(descs, packed, scales, x, q, sx, y, status=None, stream=None) -> None:
    """Device: several independent GEMVs of equal k from fp32 inputs, quantiser fused."""
    GroupedFusedCall(descs, packed, scales, x, q, sx, y, status)(stream)


def _f32(t, name):
    if t is not None and t.dtype != __import__("torch").float32:
        raise ValueError(f"{name}: expected float32")


def lowbit_rmsnorm(x, g, h, eps=1e-6, r=None, x_out=None, stream=None) -> None:
    """Device: h = RMSNorm(x + r; g) per row (r optional), x_out = x + r."""
    t, d = x.shape
    for v, nm in ((x, "x"), (g, "g"), (h, "h"), (r, "r"), (x_out, "x_out")):
        _f32(v, nm)
    _check(_lib.lowbit_rmsnorm(_dev(x, "x", 4 * t * d), _dev(r, "r", 4 * t * d), _dev(x_out, "x_out", 4 * t * d),
                               _dev(g, "g", 4 * d), t, d, eps, _dev(h, "h", 4 * t * d), _stream(stream)),
           "lowbit_rmsnorm")


def lowbit_rope_attention(qkv, pos, k_cache, v_cache, attn, rope_base=10000.0, stream=None) -> None:
    """Device: one token's rotary attention at position pos over one layer's
    caches [context, d] (writes row pos of both)."""
    context, d = k_cache.shape
    for v, nm in ((qkv, "qkv"), (k_cache, "k_cache"), (v_cache, "v_cache"), (attn, "attn")):
        _f32(v, nm)
    if d % 64 or tuple(v_cache.shape) != (context, d):
        raise ValueError("lowbit_rope_attention: caches must be [context, 64 * n_heads]")
    _check(_lib.lowbit_rope_attention(_dev(qkv, "qkv", 12 * d), d // 64, pos, context, rope_base,
                                      _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(attn, "attn", 4 * d),
                                      _stream(stream)), "lowbit_rope_attention")


def lowbit_swiglu(gate, up, a, stream=None) -> None:
    """Device: a = SiLU(gate) * up elementwise."""
    n = gate.numel()
    for v, nm in ((gate, "gate"), (up, "up"), (a, "a")):
        _f32(v, nm)
    _check(_lib.lowbit_swiglu(_dev(gate, "gate"), _dev(up, "up", 4 * n), n, _dev(a, "a", 4 * n), _stream(stream)),
           "lowbit_swiglu")


class DecodeModel:
    """Marshalled arguments of lowbit_decode_step: the model struct over device
    tensors the caller provides (embedding, norm gains, packed weights and
    scales in the C struct's order), with the key/value caches and the
    workspace allocated here as torch tensors."""

    def __init__(self, d_model, n_layers, n_heads, d_ff, vocab, context, descs, embed, norms, packed, scales,
                 norm_eps=1e-6, rope_base=10000.0):
        import torch
        if len(descs) != 6 or len(packed) != 5 * n_layers + 1 or len(scales) != len(packed):
            raise ValueError("DecodeModel: 6 descriptors and 5 * n_layers + 1 weight / scale tensors expected")
        _types(embed=(embed, _F32), norms=(norms, _F32), packed=(list(packed), _U8), scales=(list(scales), _F32))
        m = lowbit_model()
        m.d_model, m.n_layers, m.n_heads, m.d_ff, m.vocab, m.context = d_model, n_layers, n_heads, d_ff, vocab, context
        m.norm_eps, m.rope_base = norm_eps, rope_base
        for i, d in enumerate(descs):
            m.proj[i] = d
        m.embed = _dev(embed, "embed", 4 * vocab * d_model).value
        m.norms = _dev(norms, "norms", 4 * (2 * n_layers + 1) * d_model).value
        slot_desc = [descs[i % 5] for i in range(5 * n_layers)] + [descs[5]]
        self._packed = (ctypes.c_void_p * len(packed))(
            *[_dev(p, "packed", d.packed_bytes).value for p, d in zip(packed, slot_desc)])
        self._scales = (ctypes.c_void_p * len(scales))(
            *[_dev(s, "scales", 4 * d.n_scales).value for s, d in zip(scales, slot_desc)])
        m.packed = ctypes.cast(self._packed, _PP)
        m.scales = ctypes.cast(self._scales, _PP)
        self.k_cache = torch.zeros((n_layers, context, d_model), dtype=torch.float32, device="cuda")
        self.v_cache = torch.zeros_like(self.k_cache)
        m.k_cache, m.v_cache = self.k_cache.data_ptr(), self.v_cache.data_ptr()
        wb = int(_lib.lowbit_model_work_bytes(ctypes.byref(m)))
        if wb < 0:
            raise ValueError("DecodeModel: invalid model sizes or descriptors")
        self.work = torch.empty(wb, dtype=torch.uint8, device="cuda")
        m.work = self.work.data_ptr()
        self.trace_floats = int(_lib.lowbit_model_trace_floats(ctypes.byref(m)))
        self.model = m
        self._keep = (embed, norms, list(packed), list(scales))

    def step(self, state, logits, tokens=None, trace=None, stream=None, noalloc=False) -> None:
        """One step (lowbit_decode_step); noalloc=True calls
        lowbit_decode_step_noalloc, whose workspace is the library's static
        per-GPU array instead of self.work."""
        _types(state=(state, _I32), logits=(logits, _F32), tokens=(tokens, _I32), trace=(trace, _F32))
        m = self.model
        fn = _lib.lowbit_decode_step_noalloc if noalloc else _lib.lowbit_decode_step
        _check(fn(ctypes.byref(m), _dev(state, "state", 16), _dev(logits, "logits", 4 * m.vocab),
                  _dev(tokens, "tokens", 4 * m.context), _dev(trace, "trace", 4 * self.trace_floats),
                  _stream(stream)),
               "lowbit_decode_step_noalloc" if noalloc else "lowbit_decode_step")


def lowbit_calib_read(src, sink, stream=None) -> None:
    """Device: stream every 16-byte word of src (any contiguous GPU tensor,
    a multiple of 16 bytes) once; sink: a device int32/uint32 [1] (its value
    means nothing).  Time it with events for the read ceiling."""
    _types(sink=(sink, (_I32, "uint32")))
    nbytes = src.numel() * src.element_size()
    _check(_lib.lowbit_calib_read(_dev(src, "src"), nbytes, _dev(sink, "sink", 4), _stream(stream)),
           "lowbit_calib_read")


def lowbit_calib_mfma_i8(iters, sink, stream=None) -> int:
    """Device: the int8 matrix-core loop (iters iterations per wavefront);
    returns the number of int8 operations the launch does."""
    _types(sink=(sink, (_I32, "uint32")))
    _check(_lib.lowbit_calib_mfma_i8(int(iters), _dev(sink, "sink", 4), _stream(stream)), "lowbit_calib_mfma_i8")
    return int(_lib.lowbit_calib_mfma_i8_ops(int(iters)))


def lowbit_max_k(format: int) -> int:
    return int(_lib.lowbit_max_k(format))


def lowbit_abi_version() -> int:
    return int(_lib.lowbit_abi_version())


def raw_library() -> ctypes.CDLL:
    """The loaded ctypes handle (for callers that marshal arguments themselves)."""
    return _lib
