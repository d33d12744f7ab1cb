"""GPU parity of the original BitNet BitLinear forward ("Native Binary and
Ternary Transformers", 0x02B-0x02E): the Q_b = 128 quantiser
(lowbit_act_quant_v1, per token and per tensor) bit for bit against the
oracle over every launch shape of the quantiser kernels, its rejected and
zero rows; the sub-layer LayerNorm against the binary64 oracle within an
fp32 bound; and the whole layer - LayerNorm, codes, centered binary weights,
the GEMV and the GEMM - against the oracle's forward."""
import numpy as np
import pytest

import oracle
from oracle import bitnet_v1 as v1
from tests.gpu_common import TOL_ABS, TOL_REL, group_sum_slack, lib, say, to_dev

pytestmark = pytest.mark.gpu


def _v1_dev(x_dev, per_tensor, eps=1e-5):
    import torch
    t, k = x_dev.shape
    q = torch.full((t, k), 99, dtype=torch.int8, device="cuda")
    sx = torch.full((t,), -1.0, dtype=torch.float32, device="cuda")
    st = torch.zeros((1,), dtype=torch.int32, device="cuda")
    work = torch.full((2,), 12345, dtype=torch.int32, device="cuda")   # stale contents: the call clears it
    lib().lowbit_act_quant_v1(x_dev, q, sx, eps=eps, per_tensor=per_tensor, status=st, work=work)
    torch.cuda.synchronize()
    return q.cpu().numpy(), sx.cpu().numpy(), int(st.cpu()[0])


def _check(x, per_tensor, eps, q, sx, st, what):
    q_ref, sx_ref, rs = v1.act_quant_v1(x, per_tensor=per_tensor, eps=eps)
    assert (q == q_ref).all(), f"{what}: {int((q != q_ref).sum())} codes differ"
    ok = rs == 0
    assert (sx[ok].view(np.uint32) == sx_ref[ok].view(np.uint32)).all(), f"{what}: s_x differs"
    assert np.isnan(sx[~ok]).all(), what
    want = (1 if (rs == 1).any() else 0) | (2 if (rs == 2).any() else 0)
    assert st == want, f"{what}: status {st}, expected {want}"


@pytest.mark.parametrize("per_tensor", [False, True])
@pytest.mark.parametrize("t,k", [(37, 192), (9, 500), (33, 768), (5, 2048), (3, 4096), (2, 9728), (2, 20000),
                                 (7, 203), (1, 1), (300, 64)])
def test_codes_match_oracle(t, k, per_tensor):
    """Every launch shape of the quantiser: 8 / 16 / 32 / 64 lanes or a
    workgroup per row from registers, the two-pass loop, and odd k."""
    say(f"[case] act_quant_v1 t={t} k={k} per_tensor={per_tensor}")
    g = np.random.default_rng(t * 7919 + k)
    x = (g.standard_normal((t, k)) * g.uniform(0.1, 3.0, size=(t, 1))).astype(np.float32)
    q, sx, st = _v1_dev(to_dev(x), per_tensor)
    _check(x, per_tensor, 1e-5, q, sx, st, f"t={t} k={k} pt={per_tensor}")
    assert q.min() >= -128 and q.max() <= 127


def test_edge_rows():
    """Zero rows (eps = 1e-5 and eps = 0), -128 codes, NaN, Inf, a row whose
    128 max|x| overflows, a tiny row; per tensor, any of them rejects every
    row."""
    say("[case] act_quant_v1 edge rows")
    k = 256
    x = np.random.default_rng(5).standard_normal((8, k)).astype(np.float32)
    x[1] = 0.0
    x[2, 0] = -np.abs(x[2]).max() * 2          # the row's max is negative: its code is -128
    x[3, 9] = np.nan
    x[4, 100] = np.inf
    x[5, 3] = np.float32(3e37)
    x[6] = np.float32(2.0 ** -140)
    for eps in (1e-5, 0.0):
        q, sx, st = _v1_dev(to_dev(x), False, eps)
        _check(x, False, eps, q, sx, st, f"edge rows eps={eps}")
        assert q[2].min() == -128 and sx[1] == 0 and not q[1].any()
        q, sx, st = _v1_dev(to_dev(x), True, eps)
        _check(x, True, eps, q, sx, st, f"edge rows per tensor eps={eps}")
        assert not q.any() and np.isnan(sx).all() and st == 1      # the tensor's verdict: non-finite
    good = x[[0, 1, 2, 7]]
    q, sx, st = _v1_dev(to_dev(good), True, 0.0)
    _check(good, True, 0.0, q, sx, st, "per tensor, good rows, eps = 0")
    over = x[[0, 5]]                                   # finite, but 128 max|x| overflows
    q, sx, st = _v1_dev(to_dev(over), True)
    _check(over, True, 1e-5, q, sx, st, "per tensor, overflow")
    assert st == 2


@pytest.mark.parametrize("t,d", [(1, 64), (13, 192), (300, 768), (4, 4096), (2, 9728)])
def test_layernorm(t, d):
    """fp32 sums against binary64: |y - y64| <= 1e-5 (1 + |y64|) (the fp32
    mean and second moment of d terms, one division, one square root)."""
    import torch
    say(f"[case] layernorm t={t} d={d}")
    g = np.random.default_rng(d + t)
    x = (g.standard_normal((t, d)) * 2 + g.standard_normal((t, 1)) * 5).astype(np.float32)
    gain = (1 + 0.1 * g.standard_normal(d)).astype(np.float32)
    bias = (0.1 * g.standard_normal(d)).astype(np.float32)
    for gb in ((None, None), (gain, bias)):
        out = torch.empty((t, d), device="cuda")
        lib().lowbit_layernorm(to_dev(x), out, eps=1e-5, gain=None if gb[0] is None else to_dev(gb[0]),
                               bias=None if gb[1] is None else to_dev(gb[1]))
        torch.cuda.synchronize()
        ref = v1.layer_norm(x, 1e-5, *gb)
        err = np.abs(out.cpu().numpy().astype(np.float64) - ref)
        assert (err <= 1e-5 * (1 + np.abs(ref))).all(), f"layernorm t={t} d={d}: worst {err.max():.3e}"
    xi = to_dev(x)                                     # in place
    lib().lowbit_layernorm(xi, xi, eps=1e-5)
    torch.cuda.synchronize()
    assert np.abs(xi.cpu().numpy() - v1.layer_norm(x, 1e-5)).max() <= 1e-5 * (1 + np.abs(v1.layer_norm(x)).max())


@pytest.mark.parametrize("entry,scale,n,k,t", [
    ("gemv", "tensor", 768, 192, 1),
    ("gemv", "row", 192, 768, 4),
    ("gemm", "tensor", 768, 192, 8192),       # the binary model's FFN up / gate shape, 8192 tokens
    ("gemm", "row", 192, 768, 517),
    ("gemm", "group", 1024, 1024, 64),
])
def test_bitlinear_v1_forward(entry, scale, n, k, t):
    """x -> LayerNorm -> Q_b = 128 codes (per token) -> centered binary
    product, on the GPU, against the oracle's forward (binary64 LayerNorm
    rounded to fp32, then the same codes and exact product).  Where fp32 and
    binary64 put a normalised value on opposite sides of a rounding boundary
    one code moves by one; the accumulators must then differ by exactly the
    moved codes' contribution, and y by that much times s_w s_x."""
    import torch
    say(f"[case] BitNet v1 forward {entry} {scale} n={n} k={k} t={t}")
    group = 128 if scale == "group" else 0
    g = np.random.default_rng(n + k + t)
    w = (0.02 * g.standard_normal((n, k)) + 0.003).astype(np.float32)
    x = (g.standard_normal((t, k)) * 3 + 1).astype(np.float32)
    L = lib()
    d = L.lowbit_describe(L.BINARY1, L.SCALES[scale], n, k, group, L.FLAG_CENTERED)
    packed = np.empty(d.packed_bytes, np.uint8)
    scales = np.empty(d.n_scales, np.float32)
    L.lowbit_pack(d, w, packed, scales)
    xn = torch.empty((t, k), device="cuda")
    L.lowbit_layernorm(to_dev(x), xn, eps=1e-5)
    q = torch.empty((t, k), dtype=torch.int8, device="cuda")
    sx = torch.empty((t,), device="cuda")
    L.lowbit_act_quant_v1(xn, q, sx, eps=1e-5)
    y = torch.empty((t, n), device="cuda")
    acc = torch.empty((t, n, d.n_groups), dtype=torch.int32, device="cuda")
    (L.lowbit_linear if entry == "gemv" else L.lowbit_linear_batched)(d, to_dev(packed), to_dev(scales), q, sx, y, acc)
    torch.cuda.synchronize()

    xn_ref = v1.layer_norm(x, 1e-5).astype(np.float32)
    q_ref, sx_ref, rs = v1.act_quant_v1(xn_ref)
    assert (rs == 0).all()
    codes = v1.centered_binary_codes(w, scale, group)
    _, natural = oracle.weight_codes(w, "binary", scale, group)
    y32, _, acc_ref = oracle.linear(oracle.pack(codes, "binary"), oracle.pack_scales(natural, scale, n, k, group),
                                    "binary", scale, group, n, k, q_ref, sx_ref)
    qg, sxg, accg, yg = q.cpu().numpy(), sx.cpu().numpy(), acc.cpu().numpy().astype(np.int64), y.cpu().numpy()
    dq = qg.astype(np.int64) - q_ref.astype(np.int64)
    assert np.abs(dq).max() <= 1 and (dq != 0).mean() < 1e-3, f"{int((dq != 0).sum())} codes moved"
    assert (np.abs(sxg.astype(np.float64) / sx_ref - 1) <= 2e-5).all()
    # the accumulators differ exactly by the moved codes times the weight codes
    G = d.n_groups
    span = group if scale == "group" else k
    expect = acc_ref.copy()
    rows = np.nonzero(dq.any(axis=1))[0]
    for gi in range(G):
        cs = slice(gi * span, min(k, (gi + 1) * span))
        expect[rows, :, gi] += dq[rows, cs] @ codes[:, cs].T.astype(np.int64)
    assert (accg == expect).all(), "accumulators differ beyond the moved codes"
    # y: the oracle's value plus the moved codes' share (at most |s_w| s_x
    # each), the s_x difference, and for group scales the rounding slack of
    # a G-term fp32 sum taken in another order
    sw = natural.reshape(n, -1) if scale != "tensor" else np.full((n, 1), natural[0])
    moved = np.abs(dq).sum(axis=1, keepdims=True).astype(np.float64)
    bound = TOL_ABS + TOL_REL * np.abs(y32) + moved * np.abs(sw).max(axis=1)[None, :] * sx_ref[:, None] * 1.01
    bound += 2e-5 * np.abs(y32)
    if scale == "group":
        bound += group_sum_slack(expect, natural.reshape(n, -1), sxg)
    err = np.abs(yg.astype(np.float64) - y32)
    assert (err <= bound).all(), f"y: worst {err.max():.3e}"


def test_graph_replays_match_eager():
    """LayerNorm, the per-tensor Q_b = 128 codes (whose workspace a kernel
    clears, so that a replay starts from zero) and the rotated 4-bit codes,
    captured in a HIP graph: replays on a smaller-max input after a larger
    one, with eager work and synchronisations between them, equal the eager
    calls bit for bit (a stale tensor max would not)."""
    import torch
    say("[case] v1 / h4 graph replays")
    L = lib()
    t, k = 257, 768
    x = torch.empty((t, k), device="cuda")
    xn = torch.empty_like(x)
    qv = torch.empty((t, k), dtype=torch.int8, device="cuda")
    sv = torch.empty((t,), device="cuda")
    qh = torch.empty((t, k), dtype=torch.int8, device="cuda")
    sh = torch.empty((t,), device="cuda")
    work = torch.zeros(2, dtype=torch.int32, device="cuda")

    def body():
        L.lowbit_layernorm(x, xn, eps=1e-5)
        L.lowbit_act_quant_v1(x, qv, sv, per_tensor=True, work=work)
        L.lowbit_act_quant_h4(x, qh, sh)

    def inputs(seed, scale):
        g = np.random.default_rng(seed)
        x.copy_(to_dev((g.standard_normal((t, k)) * scale).astype(np.float32)))
        torch.cuda.synchronize()

    def eager():
        body()
        torch.cuda.synchronize()
        return [a.cpu().clone() for a in (xn, qv, sv, qh, sh)]

    inputs(1, 8.0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        body()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        body()
    torch.cuda.synchronize()
    for rep, (seed, scale) in enumerate([(1, 8.0), (1, 8.0), (2, 0.5), (2, 0.5), (3, 2.0)]):
        inputs(seed, scale)
        ref = eager()
        for a in (xn, qv, sv, qh, sh):
            a.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("layernorm", "v1 codes", "v1 s_x", "h4 codes", "h4 s_x"),
                              [a.cpu() for a in (xn, qv, sv, qh, sh)], ref):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager calls"
