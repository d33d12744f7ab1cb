"""Shared helpers for the GPU parity tests: run one layer through the C ABI and
through the oracle on the same seeded inputs, and compare."""
import sys

import numpy as np

import oracle

TOL_REL, TOL_ABS = 1e-5, 1e-6


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def lib():
    import bit_weight_linear_bitlinear_amd as lb
    return lb


def to_dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to("cuda", non_blocking=False) if dtype is None else t.to("cuda", dtype)


def pack_upload(w, fmt, scale, group=0, tanh=False):
    """Host pack through the library; returns (desc, packed_dev, scales_dev, packed_host, scales_host)."""
    lb = lib()
    n, k = w.shape
    d = lb.lowbit_describe(lb.FORMATS[fmt], lb.SCALES[scale], n, k, group, lb.FLAG_TANH3 if tanh else 0)
    packed = np.empty(d.packed_bytes, np.uint8)
    scales = np.empty(d.n_scales, np.float32)
    lb.lowbit_pack(d, np.ascontiguousarray(w, dtype=np.float32), packed, scales)
    return d, to_dev(packed), to_dev(scales), packed, scales


def act_quant_dev(x_dev):
    import torch
    lb = lib()
    t, k = x_dev.shape
    q = torch.empty((t, k), dtype=torch.int8, device="cuda")
    sx = torch.empty((t,), dtype=torch.float32, device="cuda")
    st = torch.zeros((1,), dtype=torch.int32, device="cuda")
    lb.lowbit_act_quant(x_dev, q, sx, st)
    return q, sx, st


def linear_dev(entry, d, packed, scales, q, sx, with_acc=True):
    import torch
    lb = lib()
    t = q.shape[0]
    y = torch.full((t, d.n), float("nan"), dtype=torch.float32, device="cuda")
    acc = torch.full((t, d.n, d.n_groups), -(2**31), dtype=torch.int32, device="cuda") if with_acc else None
    fn = lb.lowbit_linear if entry == "gemv" else lb.lowbit_linear_batched
    fn(d, packed, scales, q, sx, y, acc)
    return y, acc


def linear_fused_dev(d, packed, scales, x_dev):
    """lowbit_linear_fused on fresh (poisoned) output buffers."""
    import torch
    lb = lib()
    t = x_dev.shape[0]
    y = torch.full((t, d.n), float("nan"), dtype=torch.float32, device="cuda")
    q = torch.full((t, d.k), 99, dtype=torch.int8, device="cuda")
    sx = torch.full((t,), -1.0, dtype=torch.float32, device="cuda")
    st = torch.zeros((1,), dtype=torch.int32, device="cuda")
    lb.lowbit_linear_fused(d, packed, scales, x_dev, q, sx, y, st)
    return y, q, sx, st


def group_sum_slack(acc, scales_nat, sx):
    """Rounding-order term for group scales: y = s_x * sum_g s_w[g] acc[g] is
    a G-term fp32 sum, and two summation orders may differ by up to
    2 (G + 1) 2^-24 |s_x| sum_g |s_w[g] acc[g]| (each within (G - 1) u of the
    exact sum, plus the final products), which exceeds a bound relative to |y|
    wherever the terms cancel.  acc int64 [t, n, G], scales_nat [n, G]."""
    G = acc.shape[2]
    terms = np.abs(scales_nat.astype(np.float64)[None, :, :] * acc.astype(np.float64)).sum(axis=2)
    return 2.0 * (G + 1) * 2.0 ** -24 * np.abs(sx.astype(np.float64))[:, None] * terms


def check_y(y_gpu, y32, y64, what, slack=None):
    y_gpu = np.asarray(y_gpu, np.float32)
    err = np.abs(y_gpu.astype(np.float64) - y32.astype(np.float64))
    bound = TOL_ABS + TOL_REL * np.abs(y32.astype(np.float64))
    if slack is not None:
        bound = bound + slack
    bad = ~(err <= bound)
    assert not bad.any(), (f"{what}: {int(bad.sum())} y values out of tolerance; worst err "
                           f"{float(err.max()):.3e} at {np.unravel_index(int(err.argmax()), err.shape)}")
    # and against the binary64 evaluation of the same expression
    err64 = np.abs(y_gpu.astype(np.float64) - y64)
    bound64 = TOL_ABS + TOL_REL * np.abs(y64)
    if slack is not None:
        bound64 = bound64 + slack
    assert (err64 <= bound64).all(), what


def run_layer(w, x, fmt, scale, group, tanh, entries=("gemv", "gemm"), token_sample=None, label=""):
    """Pack, quantise and multiply through the library; check every stage
    against the oracle.  token_sample: indices of tokens the oracle recomputes
    (None = all)."""
    import torch
    say(f"[case] {label} fmt={fmt} scale={scale} group={group} tanh={tanh} W={w.shape} x={x.shape} "
        f"entries={entries}")
    d, packed, scales, ph, sh = pack_upload(w, fmt, scale, group, tanh)
    p_ref, s_ref, _, _ = oracle.quantize_and_pack(w, fmt, scale, group, tanh)
    assert (ph == p_ref).all(), f"{label}: packed bytes differ"
    assert (sh.view(np.uint32) == s_ref.view(np.uint32)).all(), f"{label}: scales differ"

    x_dev = to_dev(x)
    q, sx, st = act_quant_dev(x_dev)
    torch.cuda.synchronize()
    sel = np.arange(x.shape[0]) if token_sample is None else np.asarray(token_sample)
    q_ref, sx_ref, rs = oracle.act_quant(x[sel])
    assert (rs == 0).all()
    q_h = q.cpu().numpy()
    sx_h = sx.cpu().numpy()
    assert (q_h[sel] == q_ref).all(), f"{label}: activation codes differ"
    assert (sx_h[sel].view(np.uint32) == sx_ref.view(np.uint32)).all(), f"{label}: activation scales differ"
    assert int(st.cpu()[0]) == 0

    y32, y64, acc_ref = oracle.linear(p_ref, s_ref, fmt, scale, group, w.shape[0], w.shape[1], q_ref, sx_ref)
    out = {}
    for entry in entries:
        y, acc = linear_dev(entry, d, packed, scales, q, sx)
        torch.cuda.synchronize()
        acc_h = acc.cpu().numpy()[sel]
        assert (acc_h == acc_ref).all(), (f"{label} {entry}: int32 accumulators differ in "
                                          f"{int((acc_h != acc_ref).sum())} places")
        check_y(y.cpu().numpy()[sel], y32, y64, f"{label} {entry}")
        # the streaming kernels (no integer output) must give the same y bit for bit
        y_stream, _ = linear_dev(entry, d, packed, scales, q, sx, with_acc=False)
        torch.cuda.synchronize()
        assert torch.equal(y_stream, y), f"{label} {entry}: y without acc differs from y with acc"
        if entry == "gemv":
            # the quantiser fused into the product: the same codes, scales and y
            yf, qf, sxf, stf = linear_fused_dev(d, packed, scales, x_dev)
            torch.cuda.synchronize()
            assert torch.equal(qf, q), f"{label}: fused codes differ from lowbit_act_quant's"
            assert torch.equal(sxf.view(torch.int32), sx.view(torch.int32)), f"{label}: fused scales differ"
            assert int(stf.cpu()[0]) == 0
            assert torch.equal(yf, y), f"{label}: fused y differs from act-quant + product"
        out[entry] = (y, acc)
    if len(entries) == 2:
        a0, a1 = out["gemv"][1], out["gemm"][1]
        assert torch.equal(a0, a1), f"{label}: the two entry points' accumulators differ"
    return out
