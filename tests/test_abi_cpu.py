"""Host-side checks of the C ABI (no GPU needed): the library loads and exports
every symbol include/lowbit.h declares, descriptors and argument checks behave
as documented, and the host packer matches the oracle bit-for-bit."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import workloads
from tests.conftest import ROOT

lb = pytest.importorskip("bit_weight_linear_bitlinear_amd")

FMT = {"ternary": lb.TERNARY2, "binary": lb.BINARY1, "int4": lb.INT4}
SC = {"tensor": lb.SCALE_TENSOR, "row": lb.SCALE_ROW, "group": lb.SCALE_GROUP}


def _header_functions():
    with open(os.path.join(ROOT, "include", "lowbit.h")) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lowbit_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    names = _header_functions()
    assert set(names) >= {"lowbit_describe", "lowbit_pack", "lowbit_act_quant", "lowbit_linear",
                          "lowbit_linear_batched", "lowbit_status_string", "lowbit_max_k", "lowbit_abi_version"}
    lib = ctypes.CDLL(lb.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert lb.lowbit_abi_version() == 5


def test_describe_sizes():
    d = lb.lowbit_describe(lb.TERNARY2, lb.SCALE_GROUP, 9728, 2560, 128)
    assert (d.wpl, d.step_k, d.n_steps) == (4, 256, 10)
    assert (d.packed_bytes, d.n_groups, d.n_scales) == (9728 * 640, 20, 9728 * 20)
    d = lb.lowbit_describe(lb.BINARY1, lb.SCALE_ROW, 96, 192)
    assert (d.wpl, d.step_k, d.n_steps, d.packed_bytes, d.n_scales) == (2, 256, 1, 6 * 512, 96)
    d = lb.lowbit_describe(lb.INT4, lb.SCALE_ROW, 3840, 1280, 0, lb.FLAG_TANH3)
    assert (d.wpl, d.step_k, d.packed_bytes, d.flags) == (4, 128, 3840 * 640, 1)
    d = lb.lowbit_describe(lb.TERNARY2, lb.SCALE_TENSOR, 5, 17)
    assert (d.wpl, d.packed_bytes, d.n_scales) == (1, 256, 1)
    d = lb.lowbit_describe(lb.INT4, lb.SCALE_GROUP, 3, 200, 64)
    assert d.n_groups == 4 and d.n_scales == 16 * 4
    for fmt in ("ternary", "binary", "int4"):
        for n, k in ((1, 1), (17, 7), (3, 16), (40, 100), (16, 2560), (2, 9728), (5, 4100)):
            d = lb.lowbit_describe(FMT[fmt], 0, n, k)
            lay = oracle.layout(fmt, n, k)
            assert (d.wpl, d.n_steps, d.step_k, d.packed_bytes) == \
                (lay["wpl"], lay["n_steps"], lay["step_k"], lay["packed_bytes"]), (fmt, n, k)
            dg = lb.lowbit_describe(FMT[fmt], 2, n, k, 128)
            assert dg.n_scales == oracle.n_scales("group", n, k, 128)


@pytest.mark.parametrize("args", [
    (3, 0, 4, 4, 0, 0),          # unknown format
    (0, 3, 4, 4, 0, 0),          # unknown scale mode
    (0, 0, 0, 4, 0, 0),          # n < 1
    (0, 0, 4, 0, 0, 0),          # k < 1
    (0, 0, 4, 4, 64, 0),         # group given without group mode
    (0, 2, 4, 256, 96, 0),       # group not a multiple of 64
    (1, 2, 4, 256, 64, 0),       # binary groups need multiples of 128
    (0, 0, 4, 4, 0, 2),          # unknown flag
])
def test_describe_rejects(args):
    with pytest.raises(lb.LowbitError) as e:
        lb.lowbit_describe(*args)
    assert e.value.status == 1


def test_describe_range_bound():
    for fmt in (lb.TERNARY2, lb.BINARY1, lb.INT4):
        kmax = lb.lowbit_max_k(fmt)
        lb.lowbit_describe(fmt, 0, 1, kmax)
        with pytest.raises(lb.LowbitError) as e:
            lb.lowbit_describe(fmt, 0, 1, kmax + 1)
        assert e.value.status == 2
    # |activation code| <= 128 (the Q_b = 128 codes reach -128)
    assert lb.lowbit_max_k(lb.TERNARY2) * 128 * 64 < 2**31 <= (lb.lowbit_max_k(lb.TERNARY2) + 1) * 128 * 64
    assert lb.lowbit_max_k(lb.BINARY1) == lb.lowbit_max_k(lb.TERNARY2) == 262143
    assert lb.lowbit_max_k(lb.INT4) * 128 * 7 * 16 < 2**31 <= (lb.lowbit_max_k(lb.INT4) + 1) * 128 * 7 * 16
    assert lb.lowbit_max_k(lb.INT4) == 149796


def test_device_calls_reject_bad_arguments_before_launch():
    """Null pointers, t < 1 and tampered descriptors return E_ARG without any
    HIP call (safe on a machine with no GPU)."""
    lib = lb.raw_library()
    d = lb.lowbit_describe(lb.TERNARY2, lb.SCALE_TENSOR, 16, 64)
    one = ctypes.c_void_p(16)    # never dereferenced: every call below fails validation first
    assert lib.lowbit_act_quant(None, 1, 64, one, one, None, None) == 1
    assert lib.lowbit_act_quant(one, 0, 64, one, one, None, None) == 1
    assert lib.lowbit_linear(ctypes.byref(d), one, one, one, one, 0, one, None, None) == 1
    assert lib.lowbit_linear(ctypes.byref(d), None, one, one, one, 1, one, None, None) == 1
    assert lib.lowbit_linear_batched(ctypes.byref(d), one, one, None, one, 1, one, None, None) == 1
    for field, delta in (("wpl", 1), ("step_k", 64), ("n_steps", 1), ("packed_bytes", 256), ("n_scales", 1)):
        bad = lb.lowbit_describe(lb.TERNARY2, lb.SCALE_TENSOR, 16, 64)
        setattr(bad, field, getattr(bad, field) + delta)
        assert lib.lowbit_linear(ctypes.byref(bad), one, one, one, one, 1, one, None, None) == 1, field
    odd = ctypes.c_void_p(24)    # packed must be 16-byte aligned
    assert lib.lowbit_linear(ctypes.byref(d), odd, one, one, one, 1, one, None, None) == 1
    assert lib.lowbit_linear_batched(None, one, one, one, one, 1, one, None, None) == 1


def _pack_lib(w, fmt, scale, group=0, tanh=False):
    n, k = w.shape
    d = lb.lowbit_describe(FMT[fmt], SC[scale], n, k, group, lb.FLAG_TANH3 if tanh else 0)
    packed = np.empty(d.packed_bytes, np.uint8)
    scales = np.empty(d.n_scales, np.float32)
    lb.lowbit_pack(d, np.ascontiguousarray(w), packed, scales)
    return packed, scales


def _pack_oracle(w, fmt, scale, group=0, tanh=False):
    p, s, _, _ = oracle.quantize_and_pack(w, fmt, scale, group, tanh)
    return p, s


@pytest.mark.parametrize("wl", workloads.WORKLOADS, ids=lambda w: w.name)
def test_host_pack_matches_oracle_on_workload_shapes(wl):
    seen = set()
    for mi, m in enumerate(wl.matrices):
        if (m.n, m.k) in seen:
            continue
        seen.add((m.n, m.k))
        w = workloads.latent_weights(wl.index, 0, mi, m.n, m.k)
        p1, s1 = _pack_lib(w, wl.fmt, wl.scale, wl.group, wl.tanh_premap)
        p2, s2 = _pack_oracle(w, wl.fmt, wl.scale, wl.group, wl.tanh_premap)
        assert (p1 == p2).all(), (wl.name, m.name)
        assert (s1.view(np.uint32) == s2.view(np.uint32)).all(), (wl.name, m.name)


@pytest.mark.parametrize("fmt", ["ternary", "binary", "int4"])
@pytest.mark.parametrize("scale", ["tensor", "row", "group"])
def test_host_pack_matches_oracle_ragged(fmt, scale):
    group = (128 if fmt == "binary" else 64) if scale == "group" else 0
    for seed, (n, k) in enumerate([(1, 1), (3, 5), (17, 100), (33, 257), (5, 1000)]):
        w, _ = workloads.random_case(seed, n, k, 1)
        w[0, 0] = 0.0
        if k > 2:
            w[-1, 1] = -0.0
        for tanh in (False, True):
            p1, s1 = _pack_lib(w, fmt, scale, group, tanh)
            p2, s2 = _pack_oracle(w, fmt, scale, group, tanh)
            assert (p1 == p2).all() and (s1.view(np.uint32) == s2.view(np.uint32)).all(), (n, k, tanh)


def test_host_pack_ties_and_zero_domains():
    g = np.array([[0.25, -0.75, 0.75, -0.25, 0.5, -0.5, 0.0, 1.0]], np.float32)
    p, s = _pack_lib(g, "ternary", "tensor")
    assert s[0] == 0.5
    assert (oracle.unpack(p, "ternary", 1, 8)[0] == np.array([0, -1, 1, 0, 1, -1, 0, 1])).all()
    z = np.zeros((2, 130), np.float32)
    z[1, 129] = 1.0
    for fmt, scale, group in (("ternary", "group", 64), ("int4", "row", 0), ("binary", "group", 128)):
        p1, s1 = _pack_lib(z, fmt, scale, group)
        p2, s2 = _pack_oracle(z, fmt, scale, group)
        assert (p1 == p2).all() and (s1 == s2).all()


def test_host_pack_rejects_nonfinite_and_bad_buffers():
    w = np.ones((4, 32), np.float32)
    w[2, 7] = np.nan
    for scale in ("tensor", "row"):
        with pytest.raises(lb.LowbitError) as e:
            _pack_lib(w, "ternary", scale)
        assert e.value.status == 3
    d = lb.lowbit_describe(lb.TERNARY2, lb.SCALE_TENSOR, 4, 32)
    with pytest.raises(ValueError):
        lb.lowbit_pack(d, np.ones((4, 32), np.float32), np.empty(3, np.uint8), np.empty(1, np.float32))


def test_single_hip_runtime_in_process():
    """The binding must bind the library to torch's HIP runtime: two copies of
    libamdhip64 in one process make torch's device pointers invalid for our
    launches."""
    import re
    with open("/proc/self/maps") as f:
        paths = set(re.findall(r"\S*libamdhip64\S*", f.read()))
    assert len(paths) == 1, paths


# ------------------------------------------------------------- decode model

def _model_struct(d=256, layers=6, heads=4, ff=1024, vocab=4096, context=128):
    m = lb.lowbit_model()
    m.d_model, m.n_layers, m.n_heads, m.d_ff, m.vocab, m.context = d, layers, heads, ff, vocab, context
    m.norm_eps, m.rope_base = 1e-6, 10000.0
    shapes = [(3 * d, d), (d, d), (ff, d), (ff, d), (d, ff), (vocab, d)]
    for i, (n, k) in enumerate(shapes):
        m.proj[i] = lb.lowbit_describe(lb.TERNARY2, lb.SCALE_TENSOR, n, k)
    return m


def test_model_sizes():
    """Workspace and trace sizes of the 256-d model follow the documented
    layouts; invalid sizes report -1."""
    lib = lb.raw_library()
    m = _model_struct()
    d, ff, L = 256, 1024, 6
    up16 = lambda b: (b + 15) // 16 * 16
    want = sum(up16(b) for b in (4 * d, 4 * d, 4 * d, 12 * d, 4 * d, 4 * d, 4 * ff, 4 * ff, 4 * ff, 4 * d, 16,
                                 max(d, ff), ff))
    assert lib.lowbit_model_work_bytes(ctypes.byref(m)) == want
    # floats (padded to 4), then per layer code records of qkv, o, gate, up
    # (k = d) and down (k = ff), then the head's: 16 bytes of s_x + codes
    floats = (d + L * (12 * d + 3 * ff) + d + 3) // 4 * 4
    codes = L * (4 * (16 + up16(d)) + 16 + up16(ff)) + 16 + up16(d)
    assert lib.lowbit_model_trace_floats(ctypes.byref(m)) == floats + codes // 4
    m.d_ff = ff = 98                                          # ragged widths pad both parts
    m.proj[lb.PROJ_GATE] = lb.lowbit_describe(lb.TERNARY2, lb.SCALE_TENSOR, ff, d)
    m.proj[lb.PROJ_UP] = lb.lowbit_describe(lb.TERNARY2, lb.SCALE_TENSOR, ff, d)
    m.proj[lb.PROJ_DOWN] = lb.lowbit_describe(lb.TERNARY2, lb.SCALE_TENSOR, d, ff)
    floats = (d + L * (12 * d + 3 * ff) + d + 3) // 4 * 4
    codes = L * (4 * (16 + up16(d)) + 16 + up16(ff)) + 16 + up16(d)
    assert floats % 4 == 0 and codes % 16 == 0
    assert lib.lowbit_model_trace_floats(ctypes.byref(m)) == floats + codes // 4
    for field, bad in (("n_heads", 3), ("d_model", 250), ("context", 0), ("context", 8193), ("vocab", 0),
                       ("n_layers", 0), ("rope_base", 0.0), ("norm_eps", -1.0)):
        mb = _model_struct()
        setattr(mb, field, bad)
        assert lib.lowbit_model_work_bytes(ctypes.byref(mb)) == -1, field
    mb = _model_struct()
    mb.proj[lb.PROJ_DOWN] = lb.lowbit_describe(lb.TERNARY2, lb.SCALE_TENSOR, 256, 512)   # wrong k
    assert lib.lowbit_model_trace_floats(ctypes.byref(mb)) == -1


def test_decode_step_rejects_bad_arguments_on_the_host():
    """Every check happens before any launch: no GPU is touched."""
    lib = lb.raw_library()
    m = _model_struct()
    fake = ctypes.c_void_p(1 << 20)                          # never dereferenced: the checks fail first
    assert lib.lowbit_decode_step(ctypes.byref(m), fake, fake, None, None, None) == 1
    m.embed = m.norms = m.k_cache = m.v_cache = 1 << 20
    m.work = (1 << 20) + 8                                   # misaligned workspace
    arr = (ctypes.c_void_p * 31)(*([1 << 20] * 31))
    m.packed = ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
    m.scales = ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
    assert lib.lowbit_decode_step(ctypes.byref(m), fake, fake, None, None, None) == 1
    m.work = 1 << 20
    arr[7] = None                                            # a missing weight pointer
    assert lib.lowbit_decode_step(ctypes.byref(m), fake, fake, None, None, None) == 1


def test_act_quant_h4_rejects_bad_arguments_on_the_host():
    """Row widths without a power-of-two block of 64, widths above 65536 and
    misaligned buffers are refused before any launch."""
    lib = lb.raw_library()
    x = ctypes.c_void_p(1 << 20)                             # never dereferenced: the checks fail first
    q, sx = ctypes.c_void_p(2 << 20), ctypes.c_void_p(3 << 20)
    assert lib.lowbit_act_quant_h4(x, 1, 100, q, sx, None, None) == 1      # k % 64
    assert lib.lowbit_act_quant_h4(x, 1, 32, q, sx, None, None) == 1
    assert lib.lowbit_act_quant_h4(x, 0, 256, q, sx, None, None) == 1      # t < 1
    assert lib.lowbit_act_quant_h4(ctypes.c_void_p((1 << 20) + 4), 1, 256, q, sx, None, None) == 1
    assert lib.lowbit_act_quant_h4(x, 1, 256, ctypes.c_void_p((2 << 20) + 2), sx, None, None) == 1
    assert lib.lowbit_act_quant_h4(None, 1, 256, q, sx, None, None) == 1
    assert lib.lowbit_act_quant_h4(x, 1, 65536 + 64, q, sx, None, None) == 2   # LOWBIT_E_RANGE


def test_act_quant_a48_rejects_bad_arguments_on_the_host():
    """The a4.8 quantisers refuse bad shapes, keep counts and alignments
    before any launch."""
    lib = lb.raw_library()
    x = ctypes.c_void_p(1 << 20)                             # never dereferenced: the checks fail first
    q, sx = ctypes.c_void_p(2 << 20), ctypes.c_void_p(3 << 20)
    assert lib.lowbit_act_quant_a4(x, 0, 64, q, sx, None, None) == 1       # t < 1
    assert lib.lowbit_act_quant_a4(x, 1, 0, q, sx, None, None) == 1        # k < 1
    assert lib.lowbit_act_quant_a4(None, 1, 64, q, sx, None, None) == 1
    assert lib.lowbit_act_quant_a4(ctypes.c_void_p((1 << 20) + 2), 1, 64, q, sx, None, None) == 1
    sp = lib.lowbit_act_quant_sparse8
    assert sp(x, 1, 64, 0, q, sx, None, None) == 1                          # keep < 1
    assert sp(x, 1, 64, 65, q, sx, None, None) == 1                         # keep > k
    assert sp(x, 1, 66, 8, q, sx, None, None) == 1                          # k % 4
    assert sp(x, 0, 64, 8, q, sx, None, None) == 1                          # t < 1
    assert sp(ctypes.c_void_p((1 << 20) + 4), 1, 64, 8, q, sx, None, None) == 1
    assert sp(x, 1, 64, 8, ctypes.c_void_p((2 << 20) + 2), sx, None, None) == 1
    assert sp(x, 1, 64, 8, None, sx, None, None) == 1
    assert sp(x, 1, 32768 + 4, 8, q, sx, None, None) == 2                   # LOWBIT_E_RANGE


def _pack_centered_oracle(w, scale, group=0):
    """Centered binary codes of the BitNet v1 oracle, packed by the main
    oracle; the scales are the binary rule's mean |w|, unchanged by centering."""
    from oracle import bitnet_v1
    n, k = w.shape
    codes = bitnet_v1.centered_binary_codes(w, scale, group)
    _, natural = oracle.weight_codes(w, "binary", scale, group)
    return oracle.pack(codes, "binary"), oracle.pack_scales(natural, scale, n, k, group)


@pytest.mark.parametrize("scale", ["tensor", "row", "group"])
def test_host_pack_centered_matches_oracle(scale):
    """LOWBIT_FLAG_CENTERED: the packed bytes of the original BitNet's
    centered signs (ties to -1) and the mean |w| scales, against the oracle,
    on shifted weights (mean 0.05) where the plain rule would differ."""
    group = 128 if scale == "group" else 0
    for seed, (n, k) in enumerate([(1, 1), (3, 5), (17, 300), (33, 257), (64, 768)]):
        w, _ = workloads.random_case(seed, n, k, 1)
        w = (w + np.float32(0.05)).astype(np.float32)
        w[0, 0] = np.float32(0.05)
        d = lb.lowbit_describe(lb.BINARY1, lb.SCALES[scale], n, k, group, lb.FLAG_CENTERED)
        p1 = np.empty(d.packed_bytes, np.uint8)
        s1 = np.empty(d.n_scales, np.float32)
        lb.lowbit_pack(d, w, p1, s1)
        p2, s2 = _pack_centered_oracle(w, scale, group)
        assert (p1 == p2).all() and (s1.view(np.uint32) == s2.view(np.uint32)).all(), (scale, n, k)
    plain = _pack_lib(w, "binary", scale, group)[0]
    assert (plain != p1).any()                              # centering changed some codes


def test_centered_flag_is_binary_only():
    for fmt in (lb.TERNARY2, lb.INT4):
        with pytest.raises(lb.LowbitError):
            lb.lowbit_describe(fmt, lb.SCALE_ROW, 16, 64, 0, lb.FLAG_CENTERED)
    with pytest.raises(lb.LowbitError):
        lb.lowbit_describe(lb.BINARY1, lb.SCALE_ROW, 16, 64, 0, 4)


def test_v1_quantiser_and_layernorm_reject_bad_arguments_on_the_host():
    lib = lb.raw_library()
    x, q, sx, w = (ctypes.c_void_p(a << 20) for a in (1, 2, 3, 4))   # never dereferenced
    assert lib.lowbit_act_quant_v1(x, 1, 64, ctypes.c_float(1e-5), 1, q, sx, None, None, None) == 1   # no work
    assert lib.lowbit_act_quant_v1(x, 1, 64, ctypes.c_float(-1.0), 0, q, sx, None, None, None) == 1
    assert lib.lowbit_act_quant_v1(x, 1, 64, ctypes.c_float(float("nan")), 0, q, sx, None, None, None) == 1
    assert lib.lowbit_act_quant_v1(x, 1, 64, ctypes.c_float(1e-5), 2, q, sx, None, w, None) == 1
    assert lib.lowbit_act_quant_v1(x, 0, 64, ctypes.c_float(1e-5), 0, q, sx, None, None, None) == 1
    assert lib.lowbit_act_quant_v1(x, 1, 262144, ctypes.c_float(1e-5), 0, q, sx, None, None, None) == 2
    assert lib.lowbit_act_quant_v1(x, 1, 64, ctypes.c_float(1e-5), 1, q, sx, None,
                                   ctypes.c_void_p((4 << 20) + 2), None) == 1                   # misaligned work
    assert lib.lowbit_layernorm(x, 1, 0, ctypes.c_float(1e-5), None, None, q, None) == 1
    assert lib.lowbit_layernorm(x, 1, 64, ctypes.c_float(-1e-5), None, None, q, None) == 1
    assert lib.lowbit_layernorm(None, 1, 64, ctypes.c_float(1e-5), None, None, q, None) == 1


def _bad_dtype(fn, name):
    with pytest.raises(ValueError) as e:
        fn()
    assert f"{name}: expected dtype" in str(e.value), str(e.value)


def test_binding_rejects_wrong_dtypes():
    """Every device wrapper checks element types before any pointer reaches
    the library (a float64 x, an int32 q or a float y would otherwise be
    read or written as another type).  CPU tensors suffice: the dtype check
    comes first, so nothing touches a GPU."""
    import torch
    t, k, n = 2, 64, 16
    d = lb.lowbit_describe(lb.TERNARY2, lb.SCALE_TENSOR, n, k)
    f32 = lambda *s: torch.zeros(*s, dtype=torch.float32)
    i8 = lambda *s: torch.zeros(*s, dtype=torch.int8)
    x, q, sx, y = f32(t, k), i8(t, k), f32(t), f32(t, n)
    packed, scales = torch.zeros(d.packed_bytes, dtype=torch.uint8), f32(d.n_scales)
    acc = torch.zeros(t, n, 1, dtype=torch.int32)
    x64, q32, y64 = x.double(), q.int(), y.double()
    for quant in (lb.lowbit_act_quant, lb.lowbit_act_quant_h4, lb.lowbit_act_quant_a4):
        _bad_dtype(lambda: quant(x64, q, sx), "x")
        _bad_dtype(lambda: quant(x, q32, sx), "q")
        _bad_dtype(lambda: quant(x, q, sx.double()), "sx")
        _bad_dtype(lambda: quant(x, q, sx, status=f32(1)), "status")
    _bad_dtype(lambda: lb.lowbit_act_quant_sparse8(x64, q, sx, 3), "x")
    _bad_dtype(lambda: lb.lowbit_act_quant_sparse8(x, q32, sx, 3), "q")
    _bad_dtype(lambda: lb.lowbit_act_quant_v1(x, q32, sx), "q")
    _bad_dtype(lambda: lb.lowbit_act_quant_v1(x, q, sx, per_tensor=True, work=f32(2)), "work")
    _bad_dtype(lambda: lb.lowbit_layernorm(x64, x), "x")
    _bad_dtype(lambda: lb.lowbit_layernorm(x, x64), "out")
    for fn in (lb.lowbit_linear, lb.lowbit_linear_batched):
        _bad_dtype(lambda: fn(d, packed.to(torch.int8), scales, q, sx, y), "packed")
        _bad_dtype(lambda: fn(d, packed, scales.double(), q, sx, y), "scales")
        _bad_dtype(lambda: fn(d, packed, scales, q32, sx, y), "q")
        _bad_dtype(lambda: fn(d, packed, scales, q, sx.half(), y), "sx")
        _bad_dtype(lambda: fn(d, packed, scales, q, sx, y64), "y")
        _bad_dtype(lambda: fn(d, packed, scales, q, sx, y, acc.long()), "acc")
    _bad_dtype(lambda: lb.lowbit_linear_grouped([d], [packed], [scales], [q32], [sx], [y]), "q")
    _bad_dtype(lambda: lb.lowbit_linear_batched_grouped([d], [packed], [scales], [q], [sx], [y64]), "y")
    _bad_dtype(lambda: lb.lowbit_linear_fused(d, packed, scales, x64, q, sx, y), "x")
    _bad_dtype(lambda: lb.lowbit_linear_fused(d, packed, scales, x, q32, sx, y), "q")
    _bad_dtype(lambda: lb.lowbit_linear_grouped_fused([d], [packed], [scales], [x], [q], [sx], [y64]), "y")
    db = lb.lowbit_describe(lb.BINARY1, lb.SCALE_ROW, n, k)
    h16, g16, x16 = torch.zeros(n, dtype=torch.float16), torch.zeros(k, dtype=torch.float16), x.half()
    _bad_dtype(lambda: lb.lowbit_onebit_linear(db, packed, g16, h16, x16.bfloat16(), y), "x")
    _bad_dtype(lambda: lb.lowbit_onebit_linear(db, packed, g16.float(), h16, x16, y), "g")
    _bad_dtype(lambda: lb.lowbit_onebit_linear(db, packed, g16, h16, x16, y.half()), "y")
    _bad_dtype(lambda: lb.lowbit_linear_fused(d, packed, scales, x, q, sx, y, status=f32(1)), "status")
    descs6 = [lb.lowbit_describe(lb.TERNARY2, lb.SCALE_TENSOR, nn, kk)
              for nn, kk in ((192, 64), (64, 64), (128, 64), (128, 64), (64, 128), (100, 64))]
    pk = [torch.zeros(dd.packed_bytes, dtype=torch.uint8) for dd in descs6[:5]] + \
         [torch.zeros(descs6[5].packed_bytes, dtype=torch.int8)]
    sc = [f32(dd.n_scales) for dd in descs6[:5]] + [f32(1)]
    _bad_dtype(lambda: lb.DecodeModel(64, 1, 1, 128, 100, 8, descs6, f32(100, 64), f32(3, 64), pk, sc), "packed")
    _bad_dtype(lambda: lb.DecodeModel(64, 1, 1, 128, 100, 8, descs6, f32(100, 64).double(), f32(3, 64), pk, sc),
               "embed")


def test_decode_step_noalloc_host_checks():
    """lowbit_decode_step_noalloc: the same argument checks as
    lowbit_decode_step except that work may be NULL, and a model whose
    workspace exceeds LOWBIT_NOALLOC_WORK_BYTES is rejected with E_RANGE
    before any HIP call (no GPU is touched)."""
    lib = lb.raw_library()
    fake = ctypes.c_void_p(1 << 20)                          # never dereferenced: the checks fail first

    def filled(m, layers):
        m.embed = m.norms = m.k_cache = m.v_cache = 1 << 20
        m.work = None
        arr = (ctypes.c_void_p * (5 * layers + 1))(*([1 << 20] * (5 * layers + 1)))
        m.packed = ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
        m.scales = ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
        return arr

    m = _model_struct()
    assert lib.lowbit_decode_step_noalloc(ctypes.byref(m), fake, fake, None, None, None) == 1
    # 4096-d, FFN 65536: 36 d + 14 ff bytes of intermediates exceed 1 MiB
    big = _model_struct(d=4096, layers=1, heads=64, ff=65536, vocab=64, context=4)
    keep = filled(big, 1)
    assert lib.lowbit_model_work_bytes(ctypes.byref(big)) > lb.NOALLOC_WORK_BYTES
    assert lib.lowbit_decode_step_noalloc(ctypes.byref(big), fake, fake, None, None, None) == 2
    assert lib.lowbit_decode_step(ctypes.byref(big), fake, fake, None, None, None) == 1   # needs work
    # the 256-d model fits
    assert lib.lowbit_model_work_bytes(ctypes.byref(m)) <= lb.NOALLOC_WORK_BYTES
    keep = filled(m, 6)
    keep[3] = None                                           # a missing weight pointer is still caught
    assert lib.lowbit_decode_step_noalloc(ctypes.byref(m), fake, fake, None, None, None) == 1
    del keep


def test_calibration_calls_reject_bad_arguments_on_the_host():
    """The ceiling kernels check sizes and pointers before any launch."""
    lib = lb.raw_library()
    one = ctypes.c_void_p(1 << 20)                           # never dereferenced
    assert lib.lowbit_calib_read(None, 1024, one, None) == 1
    assert lib.lowbit_calib_read(one, 1000, one, None) == 1   # not a multiple of 16
    assert lib.lowbit_calib_read(one, 0, one, None) == 1
    assert lib.lowbit_calib_read(ctypes.c_void_p((1 << 20) + 4), 1024, one, None) == 1
    assert lib.lowbit_calib_mfma_i8(0, one, None) == 1
    assert lib.lowbit_calib_mfma_i8(10, None, None) == 1
    assert lib.lowbit_calib_mfma_i8_ops(0) == -1
