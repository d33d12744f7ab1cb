"""GPU parity of H-BitLinear's rotated 4-bit activation quantiser
(lowbit_act_quant_h4; "Native Binary and Ternary Transformers", 0x07C) and of
the layer it feeds: the codes and s_x must equal the oracle's bit for bit, and
the products on those codes keep the int8 path's bar (accumulators exact, y
within 1e-5 relative + 1e-6 absolute; with group scales plus the rounding
slack of a G-term fp32 sum taken in another order than the oracle's, since a
bound relative to |y| cannot hold where the group terms cancel).

Row widths cover every launch shape of the kernel: a wavefront per row
(up to 32 floats per lane), two wavefronts per row (two rows per workgroup,
odd token counts leaving the last one half empty), four, and sixteen for
rows above 16384; blocks of 64, 128, 256, 512, 1024 and 2048; ragged token
counts; the 4B-class widths (2560 attention, 9728 FFN) and the 4-bit QAT
model's (1280, 3584)."""
import numpy as np
import pytest

import oracle
import workloads
from oracle import hadamard as oh
from tests.gpu_common import check_y, group_sum_slack, linear_dev, pack_upload, say, to_dev

pytestmark = pytest.mark.gpu


def _h4_dev(x_dev):
    import torch
    from tests.gpu_common import lib
    t, k = x_dev.shape
    q = torch.full((t, k), 99, dtype=torch.int8, device="cuda")
    sx = torch.full((t,), -1.0, dtype=torch.float32, device="cuda")
    st = torch.zeros((1,), dtype=torch.int32, device="cuda")
    lib().lowbit_act_quant_h4(x_dev, q, sx, st)
    torch.cuda.synchronize()
    return q.cpu().numpy(), sx.cpu().numpy(), int(st.cpu()[0])


def _inputs(seed, t, k, outliers=True):
    g = np.random.default_rng(seed)
    x = g.standard_normal((t, k)).astype(np.float32)
    if outliers:   # a few channels 50x larger, the same for every token
        cols = g.choice(k, size=max(1, k // 100), replace=False)
        x[:, cols] *= np.float32(50.0)
    return x


def _check_codes(x, q, sx, st, what):
    q_ref, sx_ref, rs = oh.rotated_act_quant4(x)
    assert (q == q_ref).all(), f"{what}: {int((q != q_ref).sum())} codes differ"
    ok = rs == 0
    assert (sx[ok].view(np.uint32) == sx_ref[ok].view(np.uint32)).all(), f"{what}: s_x differs"
    assert np.isnan(sx[~ok]).all()
    want = (1 if (rs == 1).any() else 0) | (2 if (rs == 2).any() else 0)
    assert st == want, f"{what}: status {st}, expected {want}"


@pytest.mark.parametrize("t,k", [
    (1, 64), (5, 192), (3, 128), (17, 320), (2, 256), (9, 512), (4, 768), (6, 1024),     # a wavefront per row
    (3, 1280), (1, 2048), (257, 1280), (100, 576),
    (3, 2560), (16, 2560), (4, 3584), (1, 4096), (3, 6144), (1, 6912), (5, 8192),        # two per row
    (5, 9728), (2, 16384), (3, 16320),                                                   # four per row
    (1, 20480), (2, 65536), (1, 65344),                                                  # 1024 threads
])
def test_codes_match_oracle(t, k):
    say(f"[case] act_quant_h4 t={t} k={k} block={oh.block_size(k)}")
    x = _inputs(t * 100003 + k, t, k)
    q, sx, st = _h4_dev(to_dev(x))
    _check_codes(x, q, sx, st, f"t={t} k={k}")
    assert np.abs(q).max() <= 7


def test_edge_rows():
    """Zero row, NaN and Inf inputs, a pair of huge values whose butterfly sum
    overflows fp32, denormal rows (7 / m overflows), values at the rounding
    ties; the good rows of the same launch stay exact."""
    say("[case] act_quant_h4 edge rows")
    k = 512
    x = _inputs(7, 9, k, outliers=False)
    x[1] = 0.0
    x[2, 33] = np.nan
    x[3, 500] = -np.inf
    x[4, 0] = x[4, 1] = np.float32(3e38)          # x0 + x1 overflows in the first stage
    x[5] = np.float32(1e-45)
    x[6] = np.float32(0.0)
    x[6, 7] = np.float32(2.0 ** -110)             # tiny but 7 / m finite
    x[7] = np.arange(k, dtype=np.float32) - 256
    q, sx, st = _h4_dev(to_dev(x))
    _check_codes(x, q, sx, st, "edge rows")
    _, _, rs = oh.rotated_act_quant4(x)
    assert rs.tolist() == [0, 0, 1, 1, 1, 2, 0, 0, 0]
    assert sx[1] == 0 and not q[1].any()


def test_large_prefill_batch():
    """The 4-bit QAT model's prefill widths at 4096 tokens, the launch the
    bench times; every row compared (the oracle's vectorised transform covers
    them in seconds)."""
    import torch
    for k in (1280, 3584):
        say(f"[case] act_quant_h4 prefill t=4096 k={k}")
        x = workloads.activations(4, 0, 1 if k == 1280 else 4, 4096, k)
        q, sx, st = _h4_dev(to_dev(x))
        _check_codes(x, q, sx, st, f"prefill k={k}")
        torch.cuda.empty_cache()


@pytest.mark.parametrize("entry,fmt,scale,group,n,k,t", [
    ("gemv", "ternary", "group", 128, 2560, 2560, 1),     # 4B-class attention output, decode
    ("gemv", "ternary", "group", 128, 2560, 9728, 4),     # 4B-class FFN down, decode
    ("gemv", "ternary", "tensor", 0, 256, 1024, 1),       # 256-d decoder's down projection
    ("gemm", "int4", "row", 0, 1280, 3584, 512),          # 4-bit QAT FFN down, prefill
    ("gemm", "ternary", "tensor", 0, 1280, 1280, 77),     # ragged token count
])
def test_h_bitlinear_layer(entry, fmt, scale, group, n, k, t):
    """The rotated quantiser feeding the int8 products: acc equals the
    oracle's exact integer product of the oracle's codes, y within tolerance."""
    say(f"[case] H-BitLinear {entry} {fmt}/{scale} n={n} k={k} t={t}")
    w, _ = workloads.random_case(n * 7 + k, n, k, 1)
    x = _inputs(k + t, t, k)
    d, packed, scales, packed_h, scales_h = pack_upload(w, fmt, scale, group, tanh=fmt == "int4")
    import torch
    from tests.gpu_common import lib
    q = torch.empty((t, k), dtype=torch.int8, device="cuda")
    sx = torch.empty((t,), dtype=torch.float32, device="cuda")
    lib().lowbit_act_quant_h4(to_dev(x), q, sx)
    y, acc = linear_dev(entry, d, packed, scales, q, sx)
    torch.cuda.synchronize()
    q_ref, sx_ref, rs = oh.rotated_act_quant4(x)
    assert (rs == 0).all() and (q.cpu().numpy() == q_ref).all()
    y32, y64, acc_ref = oracle.linear(packed_h, scales_h, fmt, scale, group, n, k, q_ref, sx_ref)
    assert (acc.cpu().numpy().astype(np.int64) == acc_ref).all(), "accumulators differ"
    slack = None
    if scale == "group":   # a G-term fp32 sum in another order than the oracle's
        slack = group_sum_slack(acc_ref, oracle.unpack_scales(scales_h, scale, n, k, group).reshape(n, -1), sx_ref)
    check_y(y.cpu().numpy(), y32, y64, f"H-BitLinear {entry} n={n} k={k}", slack)
