"""GPU parity of OneBit's W1A16 layer ("Native Binary and Ternary
Transformers", 0x06A): the projection h * (fp16(x * g) . S^T) against the
binary64 oracle within the bound of its fp32 sums, and the whole layer (the
projection, then lowbit_layernorm over the outputs) against the oracle's.

Bound: the products are exact (+-1 times an fp16 value), the rounding is in
the fp32 sums - at most 32 terms inside one matrix-core step, then one add per
step along each of four wavefronts' chains and three adds across them - so
|y - y64| <= |h| (36 + k / 128) 2^-24 sum_k |fp16(x g)| + 2^-23 |y64|."""
import numpy as np
import pytest

from oracle import onebit
from tests.gpu_common import lib, say, to_dev

pytestmark = pytest.mark.gpu


def _layer(n, k, t, seed):
    import torch
    g = np.random.default_rng(seed)
    w = g.standard_normal((n, k)).astype(np.float32)
    w[0, :3] = [0.0, -0.0, 1.0]                          # signed zeros map to +1
    x = (g.standard_normal((t, k)) * 2).astype(np.float16)
    gv = (1 + 0.2 * g.standard_normal(k)).astype(np.float16)
    hv = (0.02 + 0.01 * g.random(n)).astype(np.float16)
    L = lib()
    d = L.lowbit_describe(L.BINARY1, L.SCALE_ROW, n, k, 0, 0)
    packed = np.empty(d.packed_bytes, np.uint8)
    scales = np.empty(d.n_scales, np.float32)
    L.lowbit_pack(d, w, packed, scales)
    y = torch.full((t, n), float("nan"), device="cuda")
    L.lowbit_onebit_linear(d, to_dev(packed), to_dev(gv), to_dev(hv), to_dev(x), y)
    torch.cuda.synchronize()
    return d, w, x, gv, hv, packed, y


def _bound(x, gv, hv, y64, k):
    l1 = np.abs(onebit.scaled_input(x, gv).astype(np.float64)).sum(axis=1, keepdims=True)
    return np.abs(hv.astype(np.float64))[None, :] * (36 + k / 128) * 2.0 ** -24 * l1 + 2.0 ** -23 * np.abs(y64)


@pytest.mark.parametrize("n,k,t", [(2560, 2560, 1), (768, 192, 4), (1000, 1000, 17), (96, 8192, 3), (64, 20000, 2),
                                   (1000, 1001, 5), (4096, 1024, 300), (16400, 256, 2),
                                   (4096, 4096, 16), (300, 2048, 33), (17, 128, 1),
                                   (4096, 1024, 2085),    # prefill with four token tiles per workgroup, t % 64 != 0
                                   (4100, 512, 4097),     # eight row tiles per wavefront (a grid of at least two
                                   (4096, 768, 4160),     # workgroups per CU), ragged n and t; two words per lane
                                   (4104, 1288, 4100),    # the same with three passes, the last ragged (k % 32 != 0)
                                   (4104, 1004, 4100)])   # k % 8 != 0: x and g staged element by element
def test_projection_matches_oracle(n, k, t):
    say(f"[case] onebit projection n={n} k={k} t={t}")
    d, w, x, gv, hv, packed, y = _layer(n, k, t, n + 3 * k + t)
    y64 = onebit.projection(x, gv, onebit.signs(w), hv)
    err = np.abs(y.cpu().numpy().astype(np.float64) - y64)
    bound = _bound(x, gv, hv, y64, k)
    assert (err <= bound).all(), f"worst {err.max():.3e}, bound there {bound.ravel()[err.argmax()]:.3e}"


@pytest.mark.parametrize("n,k,t", [(2560, 2560, 2), (768, 192, 40)])
def test_layer_with_layernorm(n, k, t):
    """y -> LayerNorm over the n outputs (in place); the projection's bound
    carried through the norm: each output moves by at most its bound / std
    plus the mean's and the deviation's share, with the norm's own fp32
    rounding (1e-5)."""
    say(f"[case] onebit layer n={n} k={k} t={t}")
    d, w, x, gv, hv, packed, y = _layer(n, k, t, 7 * n + k)
    lib().lowbit_layernorm(y, y, eps=1e-5)
    import torch
    torch.cuda.synchronize()
    s = onebit.signs(w)
    p64 = onebit.projection(x, gv, s, hv)
    ref = onebit.onebit_linear(x, gv, s, hv)
    std = p64.std(axis=1, keepdims=True)
    b = _bound(x, gv, hv, p64, k).max(axis=1, keepdims=True)
    err = np.abs(y.cpu().numpy().astype(np.float64) - ref)
    assert (err <= 3 * b / std * (1 + np.abs(ref)) + 1e-5 * (1 + np.abs(ref))).all(), f"worst {err.max():.3e}"


@pytest.mark.parametrize("t", [1, 300])
def test_graph_replays_match_eager(t):
    """The projection captured in a HIP graph (decode and prefill work
    splits): every replay, with eager work, synchronisations and a new input
    between replays, equals the eager call bit for bit."""
    import torch
    say(f"[case] onebit graph replays t={t}")
    L = lib()
    n, k = 1024, 2560
    g = np.random.default_rng(t)
    w = g.standard_normal((n, k)).astype(np.float32)
    d = L.lowbit_describe(L.BINARY1, L.SCALE_ROW, n, k)
    packed = np.empty(d.packed_bytes, np.uint8)
    L.lowbit_pack(d, w, packed, np.empty(d.n_scales, np.float32))
    pd = to_dev(packed)
    gv = to_dev((1 + 0.1 * g.standard_normal(k)).astype(np.float16))
    hv = to_dev((0.01 + 0.01 * np.abs(g.standard_normal(n))).astype(np.float16))
    x = to_dev(g.standard_normal((t, k)).astype(np.float16))
    y = torch.empty((t, n), device="cuda")

    def body():
        L.lowbit_onebit_linear(d, pd, gv, hv, x, y)

    body()
    torch.cuda.synchronize()
    ref = y.cpu().clone()
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
    for rep in range(5):
        if rep == 3:
            x.copy_(to_dev(g.standard_normal((t, k)).astype(np.float16)))
            torch.cuda.synchronize()
            body()
            torch.cuda.synchronize()
            ref = y.cpu().clone()
        y.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.cpu(), ref), f"replay {rep} differs from the eager call"
