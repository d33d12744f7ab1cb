"""GPU parity: the HIP path through the C ABI against the CPU oracle, element
by element, on the seeded workloads at their real shapes and on ragged edge
cases.  Codes, scales and int32 accumulators must match bit-for-bit; y within
1e-5 relative + 1e-6 absolute."""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_common import (act_quant_dev, check_y, linear_dev, linear_fused_dev, pack_upload, run_layer, say,
                               to_dev)

pytestmark = pytest.mark.gpu


def _distinct_matrices(wl):
    seen = {}
    for mi, m in enumerate(wl.matrices):
        seen.setdefault((m.n, m.k), (mi, m))
    return list(seen.values())


# ------------------------------------------------------------- workloads

def test_single_ternary_both_entry_points():
    wl = workloads.BY_NAME["single_ternary"]
    m = wl.matrices[0]
    w = workloads.latent_weights(wl.index, 0, 0, m.n, m.k)
    x = workloads.workload_activations(wl, 0, 0, wl.tokens[0], m.k)
    run_layer(w, x, wl.fmt, wl.scale, wl.group, wl.tanh_premap, label="single_ternary")


def test_decode_stack_all_matrices():
    wl = workloads.BY_NAME["decode_stack"]
    for layer in range(wl.layers):
        for mi, m in enumerate(wl.matrices):
            if layer >= m.count:
                continue
            w = workloads.latent_weights(wl.index, layer, mi, m.n, m.k)
            x = workloads.workload_activations(wl, layer, mi, 1, m.k)
            entries = ("gemv", "gemm") if layer == 0 else ("gemv",)
            run_layer(w, x, wl.fmt, wl.scale, wl.group, wl.tanh_premap, entries=entries,
                      label=f"decode_stack L{layer} {m.name}")


def test_binary_gqa_layer0_sampled_tokens():
    wl = workloads.BY_NAME["binary_gqa"]
    rng = np.random.default_rng(0)
    for mi, m in _distinct_matrices(wl):
        w = workloads.latent_weights(wl.index, 0, mi, m.n, m.k)
        x = workloads.workload_activations(wl, 0, mi, wl.tokens[0], m.k)
        sample = np.sort(rng.choice(wl.tokens[0], size=384, replace=False))
        sample[0], sample[-1] = 0, wl.tokens[0] - 1
        run_layer(w, x, wl.fmt, wl.scale, wl.group, wl.tanh_premap, token_sample=sample,
                  label=f"binary_gqa {m.name}")


@pytest.mark.parametrize("t", [1, 4, 16])
def test_ternary_4b_layer0(t):
    wl = workloads.BY_NAME["ternary_4b"]
    for mi, m in _distinct_matrices(wl):
        w = workloads.latent_weights(wl.index, 0, mi, m.n, m.k)
        x = workloads.workload_activations(wl, 0, mi, t, m.k)
        run_layer(w, x, wl.fmt, wl.scale, wl.group, wl.tanh_premap, label=f"ternary_4b T={t} {m.name}")


def test_int4_t4nt_layer0_sampled_tokens():
    wl = workloads.BY_NAME["int4_t4nt"]
    rng = np.random.default_rng(1)
    for mi, m in _distinct_matrices(wl):
        w = workloads.latent_weights(wl.index, 0, mi, m.n, m.k)
        x = workloads.workload_activations(wl, 0, mi, wl.tokens[0], m.k)
        sample = np.sort(rng.choice(wl.tokens[0], size=192, replace=False))
        sample[0], sample[-1] = 0, wl.tokens[0] - 1
        run_layer(w, x, wl.fmt, wl.scale, wl.group, wl.tanh_premap, token_sample=sample,
                  label=f"int4_t4nt {m.name}")


# ------------------------------------------------------- ragged / random

# (n, k, t): tails in n and k, t above 16 (several launches), t * k too large
# for the LDS activation stage (k = 4100, 4112 at t = 16), few tiles with many
# k-steps (split k-ranges)
RAGGED = [(1, 1, 1), (16, 64, 1), (17, 100, 3), (5, 257, 2), (33, 1000, 17), (130, 520, 5), (64, 4100, 16),
          (40, 384, 130), (48, 4112, 16)]


@pytest.mark.parametrize("fmt", ["ternary", "binary", "int4"])
@pytest.mark.parametrize("scale", ["tensor", "row", "group"])
def test_ragged_shapes(fmt, scale):
    for i, (n, k, t) in enumerate(RAGGED):
        group = (128 if fmt == "binary" else 64) * (1 + i % 2) if scale == "group" else 0
        w, x = workloads.random_case(100 + i, n, k, t)
        run_layer(w, x, fmt, scale, group, fmt == "int4", label=f"ragged {i}")


@pytest.mark.parametrize("fmt,k,groups", [
    ("ternary", 2560, (64, 128, 192, 256, 512, 640, 2560)),
    ("int4", 1280, (64, 128, 192, 256, 1280)),
    ("binary", 1536, (128, 256, 384, 512, 1024)),
])
def test_group_sizes(fmt, k, groups):
    """Scale groups smaller than, equal to, larger than and not aligned with a
    packed k-step, including a last group cut short by k."""
    for gi, group in enumerate(groups):
        for t in (1, 5):
            w, x = workloads.random_case(300 + gi, 200, k, t)
            run_layer(w, x, fmt, "group", group, fmt == "int4", label=f"group {group} t={t}")


def test_act_quant_edge_rows():
    """Zero rows, rows with NaN/Inf and rows whose 127/max overflows: zero
    codes, sx = NaN for the rejected ones, status bits set; good rows exact."""
    import torch
    x = np.random.default_rng(3).standard_normal((8, 203)).astype(np.float32)
    x[1] = 0.0
    x[2, 17] = np.nan
    x[3, 0] = -np.inf
    x[4] = np.float32(1e-45)
    x[5] = np.float32(5e-37)     # tiny but representable: 127 / m finite
    x[6, :] = np.arange(203, dtype=np.float32) - 101
    say("[case] act_quant edge rows")
    q, sx, st = act_quant_dev(to_dev(x))
    torch.cuda.synchronize()
    q_ref, sx_ref, rs = oracle.act_quant(x)
    qh, sxh = q.cpu().numpy(), sx.cpu().numpy()
    ok = rs == 0
    assert (qh[ok] == q_ref[ok]).all() and (sxh[ok].view(np.uint32) == sx_ref[ok].view(np.uint32)).all()
    assert (qh[~ok] == 0).all() and np.isnan(sxh[~ok]).all()
    assert rs.tolist()[2:5] == [1, 1, 2]
    assert int(st.cpu()[0]) == 3
    # aligned/vector path and scalar path agree (k % 4 != 0 above; now k % 4 == 0)
    x2 = np.random.default_rng(4).standard_normal((37, 256)).astype(np.float32) * 3
    q2, sx2, st2 = act_quant_dev(to_dev(x2))
    q2r, sx2r, _ = oracle.act_quant(x2)
    assert (q2.cpu().numpy() == q2r).all() and (sx2.cpu().numpy() == sx2r).all() and int(st2.cpu()[0]) == 0


def test_accumulator_bound_worst_case():
    """At the largest accepted k every activation code at its extreme (127,
    and -128 from the Q_b = 128 quantiser) times every weight code at its
    extreme must still be exact (the scaled int32 sums sit one step below
    2^31)."""
    import torch
    lb = pytest.importorskip("bit_weight_linear_bitlinear_amd")
    for fmt, code_w, qmax in (("ternary", 0.5, 1), ("int4", 1.0, 7), ("binary", -0.5, 1)):
        k = lb.lowbit_max_k(lb.FORMATS[fmt])
        n, t = 16, 2
        say(f"[case] worst-case accumulator fmt={fmt} k={k}")
        w = np.full((n, k), code_w, np.float32)
        w[1::2] *= -1
        x = np.ones((t, k), np.float32)
        x[1] *= -1
        d, packed, scales, _, sh = pack_upload(w, fmt, "row")
        q, sx, st = act_quant_dev(to_dev(x))
        for entry in ("gemv", "gemm"):
            y, acc = linear_dev(entry, d, packed, scales, q, sx)
            torch.cuda.synchronize()
            a = acc.cpu().numpy()[:, :, 0].astype(np.int64)
            sign_w = np.where(np.arange(n) % 2 == 0, 1, -1) * (1 if code_w > 0 else -1)
            expect = np.outer(np.array([127, -127]), sign_w * qmax) * k
            assert (a == expect).all(), (fmt, entry)
        # rows of -1 under the Q_b = 128 rule: gamma = 1, codes -128
        xv = torch.from_numpy(-np.ones((t, k), np.float32)).cuda()
        qv = torch.empty((t, k), dtype=torch.int8, device="cuda")
        sxv = torch.empty((t,), dtype=torch.float32, device="cuda")
        lb.lowbit_act_quant_v1(xv, qv, sxv)
        torch.cuda.synchronize()
        assert (qv.cpu().numpy() == -128).all()
        for entry in ("gemv", "gemm"):
            y, acc = linear_dev(entry, d, packed, scales, qv, sxv)
            torch.cuda.synchronize()
            a = acc.cpu().numpy()[:, :, 0].astype(np.int64)
            sign_w = np.where(np.arange(n) % 2 == 0, 1, -1) * (1 if code_w > 0 else -1)
            expect = np.outer(np.array([-128, -128]), sign_w * qmax) * k
            assert (a == expect).all(), (fmt, entry, "codes -128")


def test_entry_points_agree_on_random_large():
    """Moderately large random layer: GEMV and GEMM produce identical acc."""
    import torch
    w, x = workloads.random_case(7, 1000, 2048, 40)
    say("[case] gemv vs gemm random 1000x2048, t=40")
    d, packed, scales, _, _ = pack_upload(w, "ternary", "group", 128)
    q, sx, _ = act_quant_dev(to_dev(x))
    y0, a0 = linear_dev("gemv", d, packed, scales, q, sx)
    y1, a1 = linear_dev("gemm", d, packed, scales, q, sx)
    torch.cuda.synchronize()
    assert torch.equal(a0, a1)
    q_ref, sx_ref, _ = oracle.act_quant(x)
    p_ref, s_ref, _, _ = oracle.quantize_and_pack(w, "ternary", "group", 128)
    y32, y64, acc_ref = oracle.linear(p_ref, s_ref, "ternary", "group", 128, w.shape[0], 2048, q_ref, sx_ref)
    assert (a0.cpu().numpy() == acc_ref).all()
    check_y(y0.cpu().numpy(), y32, y64, "gemv")
    check_y(y1.cpu().numpy(), y32, y64, "gemm")


@pytest.mark.parametrize("fmt,scale,group,t,count", [("ternary", "group", 128, 1, 45), ("ternary", "tensor", 0, 3, 45),
                                                     ("int4", "row", 0, 16, 45), ("binary", "row", 0, 20, 45),
                                                     ("ternary", "group", 64, 5, 45), ("ternary", "tensor", 0, 1, 300)])
def test_grouped_matches_single_and_oracle(fmt, scale, group, t, count):
    """lowbit_linear_grouped over `count` matrices of equal k and mixed n (one
    launch of 45; 300 = two launches, the table holding 256) equals per-matrix
    lowbit_linear bit-for-bit in acc and y, and the oracle on a few of them."""
    import torch
    lb = pytest.importorskip("bit_weight_linear_bitlinear_amd")
    k = 640 if fmt != "binary" else 768
    ns = [16 * (1 + (i * 7) % 13) + (i % 3) for i in range(count)]
    say(f"[case] grouped fmt={fmt} scale={scale} group={group} t={t} k={k} count={len(ns)}")
    descs, packed, scales, qs, sxs, ys, accs, refs = [], [], [], [], [], [], [], []
    for i, n in enumerate(ns):
        w, x = workloads.random_case(500 + i, n, k, t)
        d, p, s, _, _ = pack_upload(w, fmt, scale, group, fmt == "int4")
        q, sx, _ = act_quant_dev(to_dev(x))
        descs.append(d); packed.append(p); scales.append(s); qs.append(q); sxs.append(sx)
        ys.append(torch.full((t, n), float("nan"), device="cuda"))
        accs.append(torch.full((t, n, d.n_groups), -7, dtype=torch.int32, device="cuda") if i % 4 != 3 else None)
        refs.append((w, x))
    lb.lowbit_linear_grouped(descs, packed, scales, qs, sxs, ys, accs)
    for i in range(len(ns)):
        y1, a1 = linear_dev("gemv", descs[i], packed[i], scales[i], qs[i], sxs[i])
        torch.cuda.synchronize()
        if scale != "group":    # integer partials: identical y whatever the k-split
            assert torch.equal(ys[i], y1), i
        else:                   # fp32 group partials may be combined in another order
            assert torch.allclose(ys[i], y1, rtol=1e-5, atol=1e-6), i
        if accs[i] is not None:
            assert torch.equal(accs[i], a1), i
    last = count - 1 if (count - 1) % 4 != 3 else count - 2    # (every fourth matrix has no integer output)
    for i in (0, 17, last):
        w, x = refs[i]
        p_ref, s_ref, _, _ = oracle.quantize_and_pack(w, fmt, scale, group, fmt == "int4")
        q_ref, sx_ref, _ = oracle.act_quant(x)
        y32, y64, acc_ref = oracle.linear(p_ref, s_ref, fmt, scale, group, w.shape[0], k, q_ref, sx_ref)
        assert (accs[i].cpu().numpy() == acc_ref).all()
        check_y(ys[i].cpu().numpy(), y32, y64, f"grouped {i}")


@pytest.mark.parametrize("fmt,t,k", [("ternary", 16, 9728), ("ternary", 7, 12208), ("ternary", 16, 9720),
                                     ("ternary", 4, 9728), ("ternary", 16, 2560), ("int4", 16, 9728),
                                     ("binary", 16, 9728), ("int4", 4, 2560), ("binary", 5, 3072)])
def test_grouped_gemv_large_stages(fmt, t, k):
    """Grouped decode GEMVs of several tokens at group-128 scales, 48
    products (three distinct matrices of 405 rows, 26 tiles each) in one
    launch, through every way a several-token stage is held:
      - larger than half a CU's LDS with one part per tile: filled in phases
        of whole ring rounds (ternary t = 16, k = 9728: 3 phases; t = 7,
        k = 12208: 2, the last step ragged; int4 and binary at t = 16,
        k = 9728, binary without the 8-waves-per-SIMD request), workgroups of
        16 tiles, the second with 6 idle wavefronts; k = 9720 (no 16-byte
        rows) stages the whole row in one 16-wavefront workgroup per CU;
      - 16-wavefront workgroups of four k-parts (ternary t = 4, k = 9728 with
        one token register; t = 16, k = 2560 with four);
      - four-wavefront workgroups (int4 t = 4, binary t = 5).
    acc equals per-matrix lowbit_linear and the oracle bit for bit, the
    streaming kernel's y equals the integer-output kernel's, and y is within
    tolerance of per-matrix calls and the oracle (group partials may be
    combined in another order)."""
    import torch
    lb = pytest.importorskip("bit_weight_linear_bitlinear_amd")
    n, count, scale, group = 405, 48, "group", 128
    say(f"[case] grouped large stage fmt={fmt} t={t} k={k} n={n} count={count}")
    mats = []
    for i in range(3):
        w, x = workloads.random_case(900 + i, n, k, t)
        d, p, s_, _, _ = pack_upload(w, fmt, scale, group, fmt == "int4")
        q, sx, _ = act_quant_dev(to_dev(x))
        mats.append((w, x, d, p, s_, q, sx))
    pick = [mats[i % 3] for i in range(count)]
    ys = [torch.full((t, n), float("nan"), device="cuda") for _ in range(count)]
    accs = [torch.full((t, n, pick[0][2].n_groups), -7, dtype=torch.int32, device="cuda") for _ in range(count)]
    lb.lowbit_linear_grouped([m[2] for m in pick], [m[3] for m in pick], [m[4] for m in pick],
                             [m[5] for m in pick], [m[6] for m in pick], ys, accs)
    ys_stream = [torch.full((t, n), float("nan"), device="cuda") for _ in range(count)]
    lb.lowbit_linear_grouped([m[2] for m in pick], [m[3] for m in pick], [m[4] for m in pick],
                             [m[5] for m in pick], [m[6] for m in pick], ys_stream)
    torch.cuda.synchronize()
    for i in range(3):
        w, x, d, p, s_, q, sx = mats[i]
        y1, a1 = linear_dev("gemv", d, p, s_, q, sx)
        p_ref, s_ref, _, _ = oracle.quantize_and_pack(w, fmt, scale, group, fmt == "int4")
        q_ref, sx_ref, _ = oracle.act_quant(x)
        y32, y64, acc_ref = oracle.linear(p_ref, s_ref, fmt, scale, group, n, k, q_ref, sx_ref)
        assert (a1.cpu().numpy() == acc_ref).all()
        for j in range(i, count, 3):
            assert torch.equal(accs[j], a1), j
            assert torch.equal(ys_stream[j], ys[j]), j
            assert torch.allclose(ys[j], y1, rtol=1e-5, atol=1e-6), j
            check_y(ys[j].cpu().numpy(), y32, y64, f"grouped large stage {j}")


@pytest.mark.parametrize("fmt,scale,group,k,t,ns", [
    ("binary", "row", 0, 192, 300, [96, 192, 768, 20, 130]),
    ("int4", "row", 0, 1280, 260, [1280, 17, 384]),
    ("ternary", "group", 128, 256, 129, [64, 300, 16]),
    ("ternary", "tensor", 0, 1000, 70, [50, 33]),              # k % 16 != 0: the general kernel, one each
    ("binary", "row", 0, 192, 77, [16 + 8 * (i % 9) for i in range(140)]),  # three launches of at most 64
    ("ternary", "group", 64, 256, 40, [16 + 16 * (i % 5) + (i % 3) for i in range(70)]),   # two launches
    ("int4", "row", 0, 128, 33, [32 + 8 * (i % 7) for i in range(65)]),
])
def test_batched_grouped_matches_single_and_oracle(fmt, scale, group, k, t, ns):
    """lowbit_linear_batched_grouped (one launch's tiles over several
    products of equal k) equals per-matrix lowbit_linear_batched bit-for-bit
    in acc and y, and the oracle on each (all at sizes the oracle runs in
    seconds)."""
    import torch
    lb = pytest.importorskip("bit_weight_linear_bitlinear_amd")
    say(f"[case] batched grouped fmt={fmt} scale={scale} group={group} k={k} t={t} count={len(ns)}")
    descs, packed, scales, qs, sxs, ys, accs, refs = [], [], [], [], [], [], [], []
    for i, n in enumerate(ns):
        w, x = workloads.random_case(700 + i, n, k, t)
        d, p, s, _, _ = pack_upload(w, fmt, scale, group, fmt == "int4")
        q, sx, _ = act_quant_dev(to_dev(x))
        descs.append(d); packed.append(p); scales.append(s); qs.append(q); sxs.append(sx)
        ys.append(torch.full((t, n), float("nan"), device="cuda"))
        accs.append(torch.full((t, n, d.n_groups), -7, dtype=torch.int32, device="cuda") if i % 3 != 2 else None)
        refs.append((w, x))
    lb.lowbit_linear_batched_grouped(descs, packed, scales, qs, sxs, ys, accs)
    ys2 = [torch.full_like(y, float("nan")) for y in ys]
    lb.lowbit_linear_batched_grouped(descs, packed, scales, qs, sxs, ys2)          # no integer outputs
    for i in range(len(ns)):
        y1, a1 = linear_dev("gemm", descs[i], packed[i], scales[i], qs[i], sxs[i])
        torch.cuda.synchronize()
        assert torch.equal(ys[i], y1) and torch.equal(ys2[i], y1), i
        if accs[i] is not None:
            assert torch.equal(accs[i], a1), i
    for i in sorted(set(range(min(len(ns), 6))) | {len(ns) - 1}):
        w, x = refs[i]
        p_ref, s_ref, _, _ = oracle.quantize_and_pack(w, fmt, scale, group, fmt == "int4")
        q_ref, sx_ref, _ = oracle.act_quant(x)
        y32, y64, acc_ref = oracle.linear(p_ref, s_ref, fmt, scale, group, w.shape[0], k, q_ref, sx_ref)
        if accs[i] is not None:
            assert (accs[i].cpu().numpy() == acc_ref).all(), i
        check_y(ys[i].cpu().numpy(), y32, y64, f"batched grouped {i}")


@pytest.mark.parametrize("scale", ["row", "tensor"])
def test_int4_grouped_gemm_many_tiles(scale):
    """A grouped int4 prefill launch of 40 products (k = 256 = two packed
    steps) with several times more workgroup tiles than the chip has CUs,
    tokens ragged (t % 256 != 0) and rows ragged (n % 256 != 0, some n below
    one tile): with the integer outputs (all products) and without, against
    single-product launches (another tile-to-workgroup map) bit for bit, and
    sampled tokens of six products against the oracle."""
    import torch
    lb = pytest.importorskip("bit_weight_linear_bitlinear_amd")
    t, k = 2085, 256
    ns = [1020 - 4 * (i % 7) if i % 4 else 100 + 64 * (i % 3) for i in range(40)]
    say(f"[case] grouped int4 gemm, many tiles, scale={scale} t={t} k={k} count={len(ns)}")
    rng = np.random.default_rng(5)
    sample = np.sort(rng.choice(t, size=64, replace=False))
    sample[0], sample[-1] = 0, t - 1
    descs, packed, scales, qs, sxs, ys, accs, xs, ws = [], [], [], [], [], [], [], [], []
    for i, n in enumerate(ns):
        w, x = workloads.random_case(900 + i, n, k, t)
        d, p, sc, _, _ = pack_upload(w, "int4", scale, 0, True)
        q, sx, _ = act_quant_dev(to_dev(x))
        descs.append(d); packed.append(p); scales.append(sc); qs.append(q); sxs.append(sx)
        ys.append(torch.full((t, n), float("nan"), device="cuda"))
        accs.append(torch.full((t, n, 1), -7, dtype=torch.int32, device="cuda"))
        xs.append(x); ws.append(w)
    lb.lowbit_linear_batched_grouped(descs, packed, scales, qs, sxs, ys, accs)
    ys2 = [torch.full_like(y, float("nan")) for y in ys]
    lb.lowbit_linear_batched_grouped(descs, packed, scales, qs, sxs, ys2)
    for i in range(len(ns)):
        y1, a1 = linear_dev("gemm", descs[i], packed[i], scales[i], qs[i], sxs[i])
        torch.cuda.synchronize()
        assert torch.equal(ys[i], y1) and torch.equal(ys2[i], y1), i
        assert torch.equal(accs[i], a1), i
    for i in (0, 1, 3, 4, 17, 39):
        p_ref, s_ref, _, _ = oracle.quantize_and_pack(ws[i], "int4", scale, 0, True)
        q_ref, sx_ref, _ = oracle.act_quant(xs[i][sample])
        y32, y64, acc_ref = oracle.linear(p_ref, s_ref, "int4", scale, 0, ns[i], k, q_ref, sx_ref)
        assert (accs[i].cpu().numpy()[sample] == acc_ref).all(), i
        check_y(ys[i].cpu().numpy()[sample], y32, y64, f"grouped many tiles {i}")


@pytest.mark.parametrize("fmt", ["ternary", "binary", "int4"])
def test_gemm_tile_shapes(fmt):
    """Prefill shapes that select each workgroup tile of the batched kernel
    (256 x 256, 128 x 192, 128 x 128 at 256 CUs), ragged in tokens, rows and k,
    checked on sampled tokens including the first and the last."""
    rng = np.random.default_rng(11)
    for i, (n, k, t) in enumerate([(3800, 272, 4000), (1250, 272, 4000), (500, 272, 300)]):
        w, x = workloads.random_case(700 + i, n, k, t)
        sample = np.sort(rng.choice(t, size=min(t, 96), replace=False))
        sample[0], sample[-1] = 0, t - 1
        run_layer(w, x, fmt, "row", 0, fmt == "int4", entries=("gemm",), token_sample=sample,
                  label=f"tile shapes n={n} k={k} t={t}")


@pytest.mark.parametrize("fmt", ["ternary", "binary", "int4"])
def test_fused_quantiser_edges(fmt):
    """The fused entry against the quantiser kernel + product.  One token (the
    quantiser runs in the product kernel's prologue): rows that are ordinary,
    with NaN, with Inf, all zero, and whose 127 / max overflows, at k from one
    word round to several (64, 1000 - ending inside a k-step -, 3072 = exactly
    one round of three words per thread; 4100, 9728, 10240 in the one round of
    ten words per thread that rows of 3073 to 10240 elements take; 12288 in
    five rounds of three), and rows the prologue does not take (k % 4 != 0, an
    x not 16-byte aligned).  Several tokens (the quantiser kernel runs first):
    the same edge rows, 17 tokens (two launches), t * k too large for the LDS
    stage.  Then the grouped call."""
    import torch
    lb = pytest.importorskip("bit_weight_linear_bitlinear_amd")
    scale = "group" if fmt == "ternary" else "row"
    group = 128 if fmt != "binary" else 0

    def compare(d, packed, scales, x, x_dev, expect_status):
        q, sx, st = act_quant_dev(x_dev)
        y, _ = linear_dev("gemv", d, packed, scales, q, sx, with_acc=False)
        yf, qf, sxf, stf = linear_fused_dev(d, packed, scales, x_dev)
        torch.cuda.synchronize()
        assert int(st.cpu()[0]) == expect_status and int(stf.cpu()[0]) == expect_status
        assert torch.equal(qf, q)
        assert torch.equal(sxf.view(torch.int32), sx.view(torch.int32))
        assert torch.equal(yf.isnan(), y.isnan())
        ok = ~y.isnan()
        assert torch.equal(yf[ok], y[ok])
        q_ref, sx_ref, rs = oracle.act_quant(x)
        good = rs == 0
        assert (qf.cpu().numpy()[good] == q_ref[good]).all()
        assert (sxf.cpu().numpy()[good].view(np.uint32) == sx_ref[good].view(np.uint32)).all()
        return yf

    def edge_rows(x):
        x[1, 7] = np.nan
        x[2, 3] = np.inf
        x[3, :] = 0.0
        x[4, :] = np.float32(1e-39)           # 127 / max overflows fp32
        return x

    # one token
    for (n, k, misalign) in [(40, 64, False), (48, 1000, False), (24, 3072, False), (33, 4100, False),
                             (20, 9728, False), (24, 10240, False), (16, 12288, False), (40, 1003, False),
                             (20, 512, True)]:
        say(f"[case] fused quantiser t=1 fmt={fmt} n={n} k={k} misaligned_x={misalign}")
        w, x5 = workloads.random_case(900 + k, n, k, 5)
        x5[0, ::97] *= 40.0                   # outliers in the ordinary row
        edge_rows(x5)
        d, packed, scales, _, _ = pack_upload(w, fmt, scale, group if scale == "group" else 0, fmt == "int4")
        for row, status in ((0, 0), (1, 1), (2, 1), (3, 0), (4, 2)):
            x = np.ascontiguousarray(x5[row:row + 1])
            x_dev = to_dev(x)
            if misalign:                      # same values, 4 bytes past a 16-byte boundary
                x_dev = torch.empty(k + 4, device="cuda")[1:1 + k].view(1, k).copy_(x_dev)
            yf = compare(d, packed, scales, x, x_dev, status)
            assert bool(yf.isnan().all()) == (status != 0)

    # several tokens
    for (n, k, t) in [(48, 1000, 6), (40, 1003, 17), (33, 4100, 16)]:
        say(f"[case] fused quantiser fmt={fmt} n={n} k={k} t={t}")
        w, x = workloads.random_case(900 + k, n, k, t)
        edge_rows(x)
        d, packed, scales, _, _ = pack_upload(w, fmt, scale, group if scale == "group" else 0, fmt == "int4")
        yf = compare(d, packed, scales, x, to_dev(x), 3)
        assert bool(yf.isnan()[1].all()) and bool(yf.isnan()[4].all())

    # grouped: 5 matrices of one k, mixed n, against the separate grouped call
    # (one token: the prologue quantiser; three: the quantiser kernel first)
    k = 2560
    for t in (1, 3):
        say(f"[case] grouped fused fmt={fmt} t={t}")
        descs, pk, sc, xs, qs, sxs, ys, yfs, qfs, sxfs = [], [], [], [], [], [], [], [], [], []
        for i, n in enumerate([2560, 64, 9728 // 8, 16, 520]):
            w, x = workloads.random_case(950 + i, n, k, t)
            d, packed, scales, _, _ = pack_upload(w, fmt, scale, group if scale == "group" else 0, fmt == "int4")
            descs.append(d); pk.append(packed); sc.append(scales); xs.append(to_dev(x))
            q, sx, _ = act_quant_dev(xs[-1])
            qs.append(q); sxs.append(sx)
            ys.append(torch.empty((t, n), device="cuda")); yfs.append(torch.full((t, n), float("nan"), device="cuda"))
            qfs.append(torch.zeros((t, k), dtype=torch.int8, device="cuda")); sxfs.append(torch.zeros(t, device="cuda"))
        lb.lowbit_linear_grouped(descs, pk, sc, qs, sxs, ys)
        st = torch.zeros(1, dtype=torch.int32, device="cuda")
        lb.lowbit_linear_grouped_fused(descs, pk, sc, xs, qfs, sxfs, yfs, st)
        torch.cuda.synchronize()
        assert int(st.cpu()[0]) == 0
        for i in range(len(descs)):
            assert torch.equal(qfs[i], qs[i]) and torch.equal(sxfs[i], sxs[i]) and torch.equal(yfs[i], ys[i]), i


def test_grouped_schedules_replay_equal_to_eager():
    """The schedules the bench times as graph replays - the int8 quantiser
    then grouped GEMVs, the grouped fused GEMVs, and grouped prefill GEMMs -
    captured once: every replay, with eager work and synchronisations
    between replays and new inputs before the last two, equals the eager
    calls bit for bit."""
    import torch
    lb = pytest.importorskip("bit_weight_linear_bitlinear_amd")
    say("[case] grouped schedules as graph replays")
    k, tp = 2560, 260
    ns = [2560, 640, 640, 2560, 1000, 48]
    descs, packed, scales = [], [], []
    for i, n in enumerate(ns):
        w, _ = workloads.random_case(900 + i, n, k, 1)
        d, p, s, _, _ = pack_upload(w, "ternary", "group", 128)
        descs.append(d); packed.append(p); scales.append(s)
    xs = [torch.empty((1, k), device="cuda") for _ in ns]
    xp = [torch.empty((tp, k), device="cuda") for _ in ns]
    q1 = [torch.empty((1, k), dtype=torch.int8, device="cuda") for _ in ns]
    s1 = [torch.empty((1,), device="cuda") for _ in ns]
    qf = [torch.empty((1, k), dtype=torch.int8, device="cuda") for _ in ns]
    sf = [torch.empty((1,), device="cuda") for _ in ns]
    qp = [torch.empty((tp, k), dtype=torch.int8, device="cuda") for _ in ns]
    sp = [torch.empty((tp,), device="cuda") for _ in ns]
    y1 = [torch.empty((1, n), device="cuda") for n in ns]
    yf = [torch.empty((1, n), device="cuda") for n in ns]
    yp = [torch.empty((tp, n), device="cuda") for n in ns]
    outs = q1 + s1 + y1 + qf + sf + yf + qp + sp + yp

    def body():
        for x, q, s in zip(xs, q1, s1):
            lb.lowbit_act_quant(x, q, s)
        lb.lowbit_linear_grouped(descs, packed, scales, q1, s1, y1)
        lb.lowbit_linear_grouped_fused(descs, packed, scales, xs, qf, sf, yf)
        for x, q, s in zip(xp, qp, sp):
            lb.lowbit_act_quant(x, q, s)
        lb.lowbit_linear_batched_grouped(descs, packed, scales, qp, sp, yp)

    def inputs(seed):
        g = np.random.default_rng(seed)
        for x in xs + xp:
            x.copy_(to_dev(g.standard_normal(tuple(x.shape)).astype(np.float32)))
        torch.cuda.synchronize()

    def eager():
        body()
        torch.cuda.synchronize()
        return [a.cpu().clone() for a in outs]

    inputs(1)
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
    for rep, seed in enumerate([1, 1, 1, 2, 3]):
        inputs(seed)
        ref = eager()
        for a in outs:
            a.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for j, (a, b) in enumerate(zip([a.cpu() for a in outs], ref)):
            assert torch.equal(a, b), f"replay {rep}: output {j} differs from the eager calls"
    assert torch.equal(yf[0].cpu(), y1[0].cpu())        # the fused schedule equals the two-call one


def test_calibration_kernels():
    """The device-ceiling kernels the bench reads its roofline fractions
    against: the read stream folds every 32-bit word of the buffer into the
    sink with XOR (checked against numpy over a 24 MiB buffer, not a multiple
    of the launch's stride), and the int8 matrix-core loop runs and reports
    its operation count (2 * 32 * 32 * 32 per MFMA, 8 per iteration per
    wavefront, 8 wavefronts per CU)."""
    import torch
    lb = pytest.importorskip("bit_weight_linear_bitlinear_amd")
    rng = np.random.default_rng(3)
    words = rng.integers(0, 2 ** 32, size=(24 << 20) // 4 + 12, dtype=np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).cuda()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    lb.lowbit_calib_read(buf, sink)
    torch.cuda.synchronize()
    assert int(sink.cpu().numpy().view(np.uint32)[0]) == int(np.bitwise_xor.reduce(words))
    ops = lb.lowbit_calib_mfma_i8(16, sink)
    torch.cuda.synchronize()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert ops == 16 * cus * 2 * 4 * 8 * 65536
