"""GPU parity of BitNet a4.8's activation codes ("Native Binary and Ternary
Transformers", 0x07B): the 4-bit input codes (lowbit_act_quant_a4) and the
sparse 8-bit intermediate codes (lowbit_act_quant_sparse8) bit for bit
against the oracle over every launch shape, keep counts from one to k, rows
whose magnitudes tie at the threshold, zero and rejected rows; the full
4096-token prefill widths on sampled rows plus properties on every row; and
the layer - sparse codes into the GEMV and the GEMM - against the oracle's
product of the oracle's codes."""
import numpy as np
import pytest

import oracle
from oracle import a48
from tests.gpu_common import check_y, lib, pack_upload, say, to_dev

pytestmark = pytest.mark.gpu


def _run(fn, x_dev, *extra):
    import torch
    t, k = x_dev.shape
    q = torch.full((t, k), 99, dtype=torch.int8, device="cuda")
    sx = torch.full((t,), -1.0, dtype=torch.float32, device="cuda")
    st = torch.zeros((1,), dtype=torch.int32, device="cuda")
    fn(x_dev, q, sx, *extra, status=st)
    torch.cuda.synchronize()
    return q.cpu().numpy(), sx.cpu().numpy(), int(st.cpu()[0])


def _check(got, ref, what):
    q, sx, st = got
    q_ref, sx_ref, rs = ref
    assert (q == q_ref).all(), f"{what}: {int((q != q_ref).sum())} codes differ"
    ok = rs == 0
    assert (sx[ok].view(np.uint32) == sx_ref[ok].view(np.uint32)).all(), f"{what}: s_x differs"
    assert np.isnan(sx[~ok]).all(), what
    want = (1 if (rs == 1).any() else 0) | (2 if (rs == 2).any() else 0)
    assert st == want, f"{what}: status {st}, expected {want}"


def _rows(t, k, seed):
    g = np.random.default_rng(seed)
    return (g.standard_normal((t, k)) * g.uniform(0.1, 3.0, size=(t, 1))).astype(np.float32)


@pytest.mark.parametrize("t,k", [(37, 192), (9, 500), (33, 768), (5, 2048), (3, 4096), (2, 9728), (2, 20000),
                                 (7, 203), (1, 1), (300, 64)])
def test_a4_codes_match_oracle(t, k):
    """Every launch shape of the quantiser (as the INT8 rule's): 8 to 64
    lanes or a workgroup per row from registers, the two-pass loop, odd k."""
    say(f"[case] act_quant_a4 t={t} k={k}")
    x = _rows(t, k, t * 31 + k)
    got = _run(lib().lowbit_act_quant_a4, to_dev(x))
    _check(got, a48.input_codes(x), f"a4 t={t} k={k}")
    assert got[0].min() >= -7 and got[0].max() <= 7


def test_a4_edge_rows():
    say("[case] act_quant_a4 edge rows")
    x = _rows(6, 256, 3)
    x[1] = 0.0
    x[2, 5] = np.nan
    x[3, 9] = -np.inf
    x[4] = np.float32(2.0 ** -140)                 # 7 / m overflows
    x[5, :4] = [3.5, -1.75, 0.25, -0.25]           # ties to even at +-0.5 and +-3.5
    x[5, 4:] = 0.0
    got = _run(lib().lowbit_act_quant_a4, to_dev(x))
    _check(got, a48.input_codes(x), "a4 edge rows")
    assert got[0][5, :4].tolist() == [7, -4, 0, 0]


def _keeps(k):
    return sorted({1, 2, max(1, k // 3), k // 2, (k * 55) // 100, k - 1, k} - {0})


@pytest.mark.parametrize("t,k", [(5, 4), (7, 64), (33, 192), (9, 1000), (4, 2560), (3, 4096), (3, 4100),
                                 (2, 9728), (2, 16384), (2, 16388), (1, 32768),
                                 (65, 192), (70, 2560), (66, 3072), (66, 3076), (65, 9728), (65, 12288)])
def test_sparse8_codes_match_oracle(t, k):
    """Every launch shape at keep counts from 1 to k: up to 64 rows, 1024
    threads per row for k <= 12288; above, 256 threads (3 or 10 float4
    each), 512 and 1024 threads (8 each); slots past k empty."""
    x = _rows(t, k, t * 7 + k)
    xd = to_dev(x)
    for keep in _keeps(k):
        say(f"[case] act_quant_sparse8 t={t} k={k} keep={keep}")
        got = _run(lib().lowbit_act_quant_sparse8, xd, keep)
        _check(got, a48.sparse_codes(x, keep), f"sparse8 t={t} k={k} keep={keep}")
        assert ((got[0] != 0).sum(axis=1) <= keep).all()


@pytest.mark.parametrize("k", [256, 2560, 9728, 20000])
def test_sparse8_ties_at_the_threshold(k):
    """Rows drawn from a few magnitudes, so that many keys tie at the
    threshold and the channel order decides which are kept; rows with runs
    of zeros and -0.0; a row of one repeated value."""
    g = np.random.default_rng(k)
    x = (g.integers(-4, 5, (6, k)) * 0.375).astype(np.float32)
    x[1, ::3] = -0.0
    x[2] = np.float32(-1.25)
    x[3, : k // 2] = 0.0
    x[4] = (g.integers(-2, 3, k) * 1e-3).astype(np.float32)
    x[5, g.integers(0, k, 7)] = 9.0                # a few outliers above a tied mass
    for rows in (x, np.tile(x, (11, 1))):             # 6 rows, and 66 (the many-row launch shapes)
        xd = to_dev(rows)
        for keep in (1, 3, 7, 8, k // 5, k // 2, k - 3):
            say(f"[case] sparse8 ties t={rows.shape[0]} k={k} keep={keep}")
            got = _run(lib().lowbit_act_quant_sparse8, xd, keep)
            _check(got, a48.sparse_codes(rows, keep), f"sparse8 ties t={rows.shape[0]} k={k} keep={keep}")


def test_sparse8_rejected_and_degenerate_rows():
    """A NaN or Inf rejects the whole row wherever it sits (also below the
    threshold); an overflowing 127 / m rejects it with status 2; zero rows get
    zero codes and s_x = 0; denormal rows keep their largest entries."""
    say("[case] sparse8 rejected rows")
    k = 512
    x = _rows(7, k, 9)
    x[0, 100] = np.nan
    x[1] = np.abs(x[1]) + 1
    x[1, 7] = 1e-3                                 # the smallest magnitude ...
    x[1, 8] = np.inf                               # ... and an Inf
    x[2] = 0.0
    x[3] = np.float32(2.0 ** -140)                 # 127 / m overflows
    x[4] = (np.arange(k) % 17 * 2.0 ** -135).astype(np.float32)   # denormals, finite 127 / m
    x[5] = -0.0
    for rows in (x, np.tile(x, (10, 1))):            # 7 rows, and 70 (the many-row launch shapes)
        for keep in (1, 64, 511, 512):
            got = _run(lib().lowbit_act_quant_sparse8, to_dev(rows), keep)
            _check(got, a48.sparse_codes(rows, keep), f"sparse8 rejected rows t={rows.shape[0]} keep={keep}")
            assert got[2] == 3 and got[1][2] == 0 and not got[0][2].any()


@pytest.mark.parametrize("k", [640, 2560, 3072])
def test_sparse8_many_rows(k):
    """Rows of up to 3072 elements (256 threads, 3 float4 each), more rows
    than stay resident at once, so that workgroups start as others end:
    every row bit for bit, real-valued rows and rows with many ties at the
    threshold."""
    t = 2600
    g = np.random.default_rng(k + 1)
    ties = (g.integers(-4, 5, (t, k)) * 0.375).astype(np.float32)
    ties[::7, ::3] = -0.0
    for name, x in (("real", _rows(t, k, 5 * k)), ("ties", ties)):
        xd = to_dev(x)
        for keep in (1, k // 2, k - 1):
            say(f"[case] sparse8 many rows t={t} k={k} {name} keep={keep}")
            got = _run(lib().lowbit_act_quant_sparse8, xd, keep)
            _check(got, a48.sparse_codes(x, keep), f"sparse8 many rows k={k} {name} keep={keep}")


@pytest.mark.parametrize("k", [2560, 9728])
def test_sparse8_prefill_widths(k):
    """The 4096-token prefill in front of the attention output (k = 2560) and
    FFN down (k = 9728) projections, in the launch shape the bench times,
    half of each row kept: 48 sampled rows (the first and last included)
    against the oracle, and on every row the properties that hold at any
    size - at most keep non-zero codes, each equal to the dense INT8 code,
    s_x the dense one, and no dropped entry larger than a kept one."""
    import torch
    t, keep = 4096, k // 2
    say(f"[case] sparse8 prefill t={t} k={k} keep={keep}")
    x = _rows(t, k, k)
    xd = to_dev(x)
    q, sx, st = _run(lib().lowbit_act_quant_sparse8, xd, keep)
    qd = torch.empty((t, k), dtype=torch.int8, device="cuda")
    sxd = torch.empty((t,), device="cuda")
    lib().lowbit_act_quant(xd, qd, sxd)
    torch.cuda.synchronize()
    qd, sxd = qd.cpu().numpy(), sxd.cpu().numpy()
    assert st == 0 and (sx.view(np.uint32) == sxd.view(np.uint32)).all()
    nz = q != 0
    assert (nz.sum(axis=1) <= keep).all() and (q[nz] == qd[nz]).all()
    a = np.abs(x)
    kept_min = np.where(nz, a, np.inf).min(axis=1)
    dropped = (qd != 0) & ~nz
    dropped_max = np.where(dropped, a, 0).max(axis=1)
    assert (dropped_max <= kept_min).all()
    rows = np.unique(np.concatenate([[0, t - 1], np.random.default_rng(k).integers(0, t, 46)]))
    _check((q[rows], sx[rows], 0), a48.sparse_codes(x[rows], keep), f"sparse8 prefill k={k} sampled rows")


@pytest.mark.parametrize("entry,fmt,scale,n,k,t", [
    ("gemv", "ternary", "tensor", 2560, 9728, 1),     # FFN down at decode
    ("gemv", "ternary", "group", 640, 2560, 4),
    ("gemm", "ternary", "tensor", 1280, 2560, 300),   # attention output at prefill
    ("gemm", "int4", "row", 256, 9728, 64),
])
def test_sparse8_layer(entry, fmt, scale, n, k, t):
    """Sparse codes as the product's input: the accumulators equal the
    oracle's exact product of the oracle's codes, y its epilogue."""
    import torch
    say(f"[case] sparse8 layer {entry} {fmt} {scale} n={n} k={k} t={t}")
    group = 128 if scale == "group" else 0
    g = np.random.default_rng(n + k + t)
    w = (0.02 * g.standard_normal((n, k))).astype(np.float32)
    x = _rows(t, k, n + t)
    keep = (k * 55) // 100
    d, pd, sd, _, _ = pack_upload(w, fmt, scale, group, fmt == "int4")
    L = lib()
    q = torch.empty((t, k), dtype=torch.int8, device="cuda")
    sx = torch.empty((t,), device="cuda")
    L.lowbit_act_quant_sparse8(to_dev(x), q, sx, keep)
    y = torch.empty((t, n), device="cuda")
    acc = torch.empty((t, n, d.n_groups), dtype=torch.int32, device="cuda")
    (L.lowbit_linear if entry == "gemv" else L.lowbit_linear_batched)(d, pd, sd, q, sx, y, acc)
    torch.cuda.synchronize()
    q_ref, sx_ref, rs = a48.sparse_codes(x, keep)
    assert (rs == 0).all() and (q.cpu().numpy() == q_ref).all()
    p_ref, s_ref, _, _ = oracle.quantize_and_pack(w, fmt, scale, group, fmt == "int4")
    y32, y64, acc_ref = oracle.linear(p_ref, s_ref, fmt, scale, group, n, k, q_ref, sx_ref)
    assert (acc.cpu().numpy() == acc_ref).all()
    slack = None
    if scale == "group":
        from tests.gpu_common import group_sum_slack
        _, natural = oracle.weight_codes(w, fmt, scale, group, fmt == "int4")
        slack = group_sum_slack(acc_ref, natural.reshape(n, -1), sx_ref)
    check_y(y.cpu().numpy(), y32, y64, f"sparse8 layer {entry}", slack)


def test_a48_graph_replays_match_eager():
    """The a4.8 quantisers feeding the products, captured in a HIP graph on a
    side stream: every replay (with eager work and synchronisations between
    replays, and a changed input before the last two) equals the eager calls
    bit for bit."""
    import torch
    say("[case] a4.8 graph replays")
    L = lib()
    t, k, n = 300, 2560, 640
    g = np.random.default_rng(21)
    w = (0.02 * g.standard_normal((n, k))).astype(np.float32)
    d, pd, sd, _, _ = pack_upload(w, "ternary", "row", 0)
    x = to_dev(_rows(t, k, 5))
    q8 = torch.empty((t, k), dtype=torch.int8, device="cuda")
    s8 = torch.empty((t,), device="cuda")
    q4 = torch.empty((1, k), dtype=torch.int8, device="cuda")
    s4 = torch.empty((1,), device="cuda")
    y8 = torch.empty((t, n), device="cuda")
    y4 = torch.empty((1, n), device="cuda")

    def body():
        L.lowbit_act_quant_sparse8(x, q8, s8, k // 2)
        L.lowbit_linear_batched(d, pd, sd, q8, s8, y8)
        L.lowbit_act_quant_a4(x[:1], q4, s4)
        L.lowbit_linear(d, pd, sd, q4, s4, y4)

    def eager():
        body()
        torch.cuda.synchronize()
        return [a.cpu().clone() for a in (q8, s8, y8, q4, s4, y4)]

    ref = eager()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        body()                                            # warm-up on the capturing stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        body()
    torch.cuda.synchronize()
    for rep in range(5):
        if rep == 3:                                      # a new input: the replay must follow it
            x.copy_(to_dev(_rows(t, k, 6)))
            torch.cuda.synchronize()
            ref = eager()
        for a in (q8, s8, y8, q4, s4, y4):
            a.zero_()                                     # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [a.cpu() for a in (q8, s8, y8, q4, s4, y4)]
        for name, a, b in zip(("q8", "s8", "y8", "q4", "s4", "y4"), got, ref):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager calls"
