"""GPU parity of the decode step of the 256-d ternary decoder (the add/sub-only
engine's quick-start model with the decode stack's projections) against the
CPU oracle (oracle/model.py), through the C ABI.

* The step's operations on their own (lowbit_rmsnorm, lowbit_rope_attention,
  lowbit_swiglu) on seeded inputs, element by element, with tolerances derived
  from their fp32 arithmetic.
* Whole steps, stage by stage (the check that decides parity): every stage
  of the step is held against the oracle applied to the GPU's own traced
  input of that stage.  Each BitLinear's int8 codes and s_x are bit-exact
  against the oracle's quantiser of its traced fp32 input, its int32
  accumulators (the library's product rerun on those codes with the integer
  output) bit-exact against the oracle's integer product, and its fp32
  output within 1e-5 relative + 1e-6 absolute of the oracle's epilogue; the
  residual adds are bit-exact fp32 sums; the fused RMSNorm and SwiGLU
  prologues, the rotary embedding and the attention are element-wise within
  bounds derived from their fp32 arithmetic; the next token is the argmax of
  the GPU's logits.
* Whole steps, teacher-forced over a seeded prompt, against the oracle run
  independently from the same seeded weights and tokens (a trajectory smoke
  check on top of the stage-by-stage one).  Up to the first
  quantised activation the two agree to fp32 rounding; after it, a value that
  the GPU (fp32) and the oracle (binary64, rounded to fp32) place on opposite
  sides of a rounding boundary moves one int8 code by one step, which moves the
  products by a few 1e-3 of their norm (the engine's README describes the same
  effect for its C++ runtime against its PyTorch model).  The bounds below are
  that, with the greedy token equal unless the oracle's top two logits are
  closer than the observed logit error.
* The captured graph of a step replays token after token, identical to eager
  steps; positions outside the context and tokens outside the vocabulary.
"""
import ctypes

import numpy as np
import pytest

import oracle
import workloads
from oracle import model as om
from tests.gpu_common import say

pytestmark = pytest.mark.gpu

CFG = workloads.DECODE_MODEL
# decode_stack matrix index of each projection slot (qkv, o, gate, up, down), head
_MI = {0: 0, 1: 1, 2: 3, 3: 2, 4: 4}
HEAD_MI = 5


def _lb():
    return pytest.importorskip("bit_weight_linear_bitlinear_amd")


def _latent(layer, slot, n, k):
    mi = _MI[slot] if slot < 5 else HEAD_MI
    return workloads.latent_weights(workloads.BY_NAME["decode_stack"].index, layer, mi, n, k)


def _shapes(d, ff, vocab):
    return [(3 * d, d), (d, d), (ff, d), (ff, d), (d, ff), (vocab, d)]


def _build_pair(d, L, H, ff, V, C, latent):
    import torch
    lb = _lb()
    shapes = _shapes(d, ff, V)
    descs = [lb.lowbit_describe(lb.TERNARY2, lb.SCALE_TENSOR, n, k) for n, k in shapes]
    embed = workloads.decode_model_embedding(V, d)
    norms = workloads.decode_model_norms(L, d)
    g_packed, g_scales, o_packed, o_scales = [], [], [], []
    for layer in range(L + 1):
        for slot in (range(5) if layer < L else [5]):
            n, k = shapes[slot]
            w = latent(layer if slot < 5 else 0, slot, n, k)
            pk = np.empty(descs[slot].packed_bytes, np.uint8)
            sc = np.empty(descs[slot].n_scales, np.float32)
            lb.lowbit_pack(descs[slot], w, pk, sc)
            g_packed.append(torch.from_numpy(pk).cuda())
            g_scales.append(torch.from_numpy(sc).cuda())
            opk, osc, _, _ = oracle.quantize_and_pack(w, "ternary", "tensor")
            o_packed.append(opk)
            o_scales.append(osc)
    gm = lb.DecodeModel(d, L, H, ff, V, C, descs, torch.from_numpy(embed).cuda(), torch.from_numpy(norms).cuda(),
                        g_packed, g_scales)
    om_ = om.Model(d, L, H, ff, V, C, embed, norms, o_packed, o_scales)
    return gm, om_


@pytest.fixture(scope="module")
def model_pair():
    """The GPU model (packed by the library) and the oracle model (packed by
    the oracle) from the same seeded latent weights, embedding and gains: the
    256-d model, whose step runs in the fused form (norms and SwiGLU inside
    the products' quantiser prologues)."""
    return _build_pair(*(CFG[k] for k in ("d", "layers", "heads", "d_ff", "vocab", "context")), _latent)


@pytest.fixture(scope="module")
def small_pair():
    """An irregular small model (one head, an FFN width that is not a multiple
    of 4) whose step takes the general form, every operation its own launch."""
    def latent(layer, slot, n, k):
        return workloads.random_case(1200 + 7 * layer + slot, n, k, 1)[0]
    return _build_pair(64, 2, 1, 98, 300, 16, latent)


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


# ------------------------------------------------------------ single ops

def test_rmsnorm_op():
    """Rows of N(0, 1), a row of scale 1e-3 (mean of squares 1e-6, where eps
    matters), widths 256, 1000 and 4096.  Residual add exact (one fp32 add);
    h within 1e-5 relative per element: fp32 sums of <= 4096 squares, one
    square root, two products."""
    import torch
    lb = _lb()
    rng = np.random.default_rng(11)
    for d in (256, 1000, 4096):
        say(f"[case] rmsnorm d={d}")
        x = rng.standard_normal((5, d)).astype(np.float32)
        x[3] *= np.float32(1e-3)
        r = rng.standard_normal((5, d)).astype(np.float32)
        r[3] *= np.float32(1e-3)
        g = (1.0 + 0.1 * rng.standard_normal(d)).astype(np.float32)
        xd, rd, gd = (torch.from_numpy(a).cuda() for a in (x, r, g))
        h = torch.empty_like(xd)
        xo = torch.empty_like(xd)
        lb.lowbit_rmsnorm(xd, gd, h, eps=1e-6, r=rd, x_out=xo)
        h0 = torch.empty_like(xd)
        lb.lowbit_rmsnorm(xd, gd, h0, eps=1e-6)
        torch.cuda.synchronize()
        v = x + r                                            # fp32, as the kernel adds
        assert np.array_equal(xo.cpu().numpy(), v)
        for got, src in ((h.cpu().numpy(), v), (h0.cpu().numpy(), x)):
            ref = om.rmsnorm(src, g, eps=1e-6)
            assert np.all(np.abs(got - ref) <= 1e-5 * np.abs(ref) + 1e-30), d


@pytest.mark.parametrize("heads", [1, 4, 8])
def test_rope_attention_op(heads):
    """Caches pre-filled with seeded rows below the position and NaN above it
    (never read); the key and value land at the position (the key rotated
    in binary64 and rounded once: 1e-6 relative to the pair's size); the
    output within 1e-5 of max|v| (fp32 scores over 64 terms, fp32 softmax
    over <= 128 positions)."""
    import torch
    lb = _lb()
    d, C = 64 * heads, 128
    rng = np.random.default_rng(20 + heads)
    for pos in (0, 1, 63, 64, 127):
        say(f"[case] rope attention heads={heads} pos={pos}")
        kc = np.full((C, d), np.nan, np.float32)
        vc = np.full((C, d), np.nan, np.float32)
        kc[:pos] = rng.standard_normal((pos, d)).astype(np.float32)
        vc[:pos] = rng.standard_normal((pos, d)).astype(np.float32)
        qkv = (2.0 * rng.standard_normal(3 * d)).astype(np.float32)
        kd, vd, qd = (torch.from_numpy(a).cuda() for a in (kc, vc, qkv))
        out = torch.empty(d, device="cuda")
        lb.lowbit_rope_attention(qd, pos, kd, vd, out)
        torch.cuda.synchronize()
        k_new = om.rope(qkv[d:2 * d], pos, heads)
        kg, vg = kd.cpu().numpy(), vd.cpu().numpy()
        kk = qkv[d:2 * d].astype(np.float64).reshape(heads, 2, 32)
        hyp = np.hypot(kk[:, 0], kk[:, 1])                   # length of each rotated pair
        pair = np.stack([hyp, hyp], axis=1).reshape(-1)      # dims i and i + 32 of each head
        assert np.all(np.abs(kg[pos] - k_new) <= 1e-6 * pair + 1e-30)
        assert np.array_equal(vg[pos], qkv[2 * d:])
        assert np.isnan(kg[pos + 1:]).all() and np.isnan(vg[pos + 1:]).all()
        kref = np.concatenate([kc[:pos].astype(np.float64), k_new[None]], axis=0)
        vref = np.concatenate([vc[:pos].astype(np.float64), qkv[None, 2 * d:].astype(np.float64)], axis=0)
        ref = om.attend(om.rope(qkv[:d], pos, heads), kref, vref, heads)
        got = out.cpu().numpy()
        assert np.all(np.abs(got - ref) <= 1e-5 * np.abs(vref).max()), (heads, pos)


def test_swiglu_op():
    """SiLU(gate) * up against binary64: fp32 exp, add, divide, multiply
    (a few ulp): 1e-6 relative per element, plus the extremes (+-80, 0)."""
    import torch
    lb = _lb()
    rng = np.random.default_rng(30)
    for n in (1024, 100003):
        gate = (3.0 * rng.standard_normal(n)).astype(np.float32)
        gate[:5] = [0.0, 80.0, -80.0, 1e-30, -1e-30]
        up = rng.standard_normal(n).astype(np.float32)
        gd, ud = torch.from_numpy(gate).cuda(), torch.from_numpy(up).cuda()
        a = torch.empty_like(gd)
        lb.lowbit_swiglu(gd, ud, a)
        torch.cuda.synchronize()
        ref = om.swiglu(gate, up)
        got = a.cpu().numpy()
        assert np.all(np.abs(got - ref) <= 1e-6 * np.abs(ref) + 1e-37), n
        assert got[0] == 0.0


# ------------------------------------------------------------ whole steps

def _state(tok, pos):
    import torch
    return torch.tensor([tok, pos, 0, 0], dtype=torch.int32, device="cuda")


def _split_trace(tr, d, L, ff):
    """The trace's float part and an accessor of its code records (layout in
    include/lowbit.h, lowbit_model_trace_floats): code(layer, slot) -> (int8
    codes [k], s_x as a float32 scalar); layer L is the head."""
    nf = d + L * (12 * d + 3 * ff) + d
    raw = tr[(nf + 3) // 4 * 4:].view(np.uint8)
    rec = lambda k: 16 + (k + 15) // 16 * 16
    per_layer = 4 * rec(d) + rec(ff)

    def code(layer, slot):
        off = L * per_layer if layer >= L else layer * per_layer + slot * rec(d)
        k = ff if (layer < L and slot == 4) else d
        return raw[off + 16:off + 16 + k].view(np.int8).copy(), raw[off:off + 4].view(np.float32)[0]
    return tr[:nf], code


def _bits(a):
    return np.asarray(a, np.float32).view(np.uint32)


@pytest.mark.parametrize("which", ["model_pair", "small_pair"])
def test_decode_step_stages_exact(which, request):
    """Twelve teacher-forced steps; at each, every stage against the oracle
    applied to the GPU's own traced input of that stage:
      - each of the 5 L + 1 BitLinears: codes and s_x bit-exact against
        oracle.act_quant of its traced input; int32 accumulators bit-exact
        against the oracle's integer product (the library's GEMV rerun on the
        traced codes with its integer output); y within 1e-5 relative + 1e-6
        absolute of the oracle's fp32 epilogue, and of its binary64 twin;
      - residual adds x_mid = x + o and x_out = x_mid + down bit-exact (one
        fp32 add each);
      - the fused RMSNorm prologues (h, h2, the final norm) within 1e-5
        relative per element of the binary64 norm of the GPU's traced
        residual stream (fp32 sums of <= 4096 squares, one square root, two
        products), the SwiGLU prologue within 1e-6 relative (fp32 exp, add,
        divide, multiply);
      - rotated q and k within 1e-6 of each pair's length; the cache rows at
        the position equal the traced key and value; the attention output
        within 1e-5 of max |v| of the binary64 attention over the GPU's
        cache rows 0 .. pos;
      - the state's next token is the argmax of the GPU's logits."""
    import torch
    lb = _lb()
    gm, om_ = request.getfixturevalue(which)
    d, L, H, ff, V = om_.d, om_.n_layers, om_.n_heads, om_.d_ff, om_.vocab
    g_packed, g_scales = gm._keep[2], gm._keep[3]
    prompt = workloads.decode_model_tokens(12, V)
    gm.k_cache.zero_()
    gm.v_cache.zero_()
    ls = 12 * d + 3 * ff
    shapes = _shapes(d, ff, V)
    names = ["h", "qkv", "q", "k", "attn", "o", "x_mid", "h2", "gate", "up", "a", "down", "x_out"]
    widths = [d, 3 * d, d, d, d, d, d, d, ff, ff, ff, d, d]
    worst = {"y_rel": 0.0, "norm_rel": 0.0, "swiglu_rel": 0.0}
    n_products = 0

    def bitlinear_stage(tag, layer, slot, x_in, y_gpu, code):
        nonlocal n_products
        q_g, sx_g = code(layer, slot if layer < L else 5)
        n, k = shapes[slot if layer < L else 5]
        q_ref, sx_ref, rs = oracle.act_quant(np.asarray(x_in, np.float32).reshape(1, k))
        assert rs[0] == 0, tag
        assert np.array_equal(q_g, q_ref[0]), f"{tag}: codes differ"
        assert _bits(sx_g) == _bits(sx_ref[0]), f"{tag}: s_x differs"
        pk, sc = om_.proj(layer, slot if layer < L else 0)
        y32, y64, acc_ref = oracle.linear(pk, sc, "ternary", "tensor", 0, n, k, q_ref, sx_ref)
        for ref in (y32[0], y64[0]):
            err = np.abs(np.asarray(y_gpu, np.float64) - ref)
            assert np.all(err <= 1e-6 + 1e-5 * np.abs(ref)), f"{tag}: y out of tolerance"
        worst["y_rel"] = max(worst["y_rel"], float((np.abs(y_gpu - y32[0]) / (1e-6 + 1e-5 * np.abs(y32[0]))).max()))
        # the integer product of the step's own codes, through the library's GEMV
        i = 5 * layer + slot if layer < L else 5 * L
        qd = torch.from_numpy(q_g.reshape(1, k)).cuda()
        sxd = torch.from_numpy(np.array([sx_g], np.float32)).cuda()
        yd = torch.empty((1, n), device="cuda")
        accd = torch.empty((1, n, 1), dtype=torch.int32, device="cuda")
        lb.lowbit_linear(gm.model.proj[slot if layer < L else 5], g_packed[i], g_scales[i], qd, sxd, yd, accd)
        torch.cuda.synchronize()
        assert np.array_equal(accd.cpu().numpy(), acc_ref), f"{tag}: accumulators differ"
        n_products += 1

    def norm_stage(tag, got, x, g):
        ref = om.rmsnorm(x, g)
        rel = np.abs(np.asarray(got, np.float64) - ref) / (np.abs(ref) + 1e-30)
        worst["norm_rel"] = max(worst["norm_rel"], float(rel.max()))
        assert np.all(rel <= 1e-5), f"{tag}: RMSNorm out of its fp32 bound"

    for pos, tok in enumerate(prompt):
        say(f"[case] {which} decode step pos={pos} token={tok} (stage by stage)")
        st = _state(int(tok), pos)
        logits = torch.empty(V, device="cuda")
        trace = torch.full((gm.trace_floats,), float("nan"), device="cuda")
        gm.step(st, logits, trace=trace)
        torch.cuda.synchronize()
        tr, code = _split_trace(trace.cpu().numpy(), d, L, ff)
        lg = logits.cpu().numpy()
        kc, vc = gm.k_cache.cpu().numpy(), gm.v_cache.cpu().numpy()
        s = st.cpu().numpy()
        assert s.tolist() == [int(np.flatnonzero(lg == lg.max())[0]), pos + 1, 0, 0]
        x = tr[:d]
        assert np.array_equal(x, om_.embed[tok])
        for l in range(L):
            off = d + l * ls
            t = {}
            for nm, w in zip(names, widths):
                t[nm] = tr[off:off + w]
                off += w
            tag = f"pos {pos} layer {l}"
            norm_stage(f"{tag} h", t["h"], x, om_.norms[2 * l])
            bitlinear_stage(f"{tag} qkv", l, 0, t["h"], t["qkv"], code)
            qkv = t["qkv"]
            kk = qkv[d:2 * d].astype(np.float64).reshape(H, 2, 32)
            hyp = np.hypot(kk[:, 0], kk[:, 1])
            qq = qkv[:d].astype(np.float64).reshape(H, 2, 32)
            hq = np.hypot(qq[:, 0], qq[:, 1])
            pair_k = np.stack([hyp, hyp], axis=1).reshape(-1)
            pair_q = np.stack([hq, hq], axis=1).reshape(-1)
            assert np.all(np.abs(t["q"] - om.rope(qkv[:d], pos, H)) <= 1e-6 * pair_q + 1e-30), f"{tag} q rot"
            assert np.all(np.abs(t["k"] - om.rope(qkv[d:2 * d], pos, H)) <= 1e-6 * pair_k + 1e-30), f"{tag} k rot"
            assert np.array_equal(kc[l, pos], t["k"]) and np.array_equal(vc[l, pos], qkv[2 * d:]), f"{tag} cache"
            ref_attn = om.attend(t["q"], kc[l, :pos + 1], vc[l, :pos + 1], H)
            assert np.all(np.abs(t["attn"] - ref_attn) <= 1e-5 * np.abs(vc[l, :pos + 1]).max()), f"{tag} attn"
            bitlinear_stage(f"{tag} o", l, 1, t["attn"], t["o"], code)
            assert np.array_equal(t["x_mid"], x + t["o"]), f"{tag} x_mid"
            norm_stage(f"{tag} h2", t["h2"], t["x_mid"], om_.norms[2 * l + 1])
            bitlinear_stage(f"{tag} gate", l, 2, t["h2"], t["gate"], code)
            bitlinear_stage(f"{tag} up", l, 3, t["h2"], t["up"], code)
            ref_a = om.swiglu(t["gate"], t["up"])
            rel = np.abs(t["a"] - ref_a) / (np.abs(ref_a) + 1e-37)
            worst["swiglu_rel"] = max(worst["swiglu_rel"], float(rel.max()))
            assert np.all(np.abs(t["a"] - ref_a) <= 1e-6 * np.abs(ref_a) + 1e-37), f"{tag} SwiGLU"
            bitlinear_stage(f"{tag} down", l, 4, t["a"], t["down"], code)
            assert np.array_equal(t["x_out"], t["x_mid"] + t["down"]), f"{tag} x_out"
            x = t["x_out"]
        hf = tr[d + L * ls:d + L * ls + d]
        norm_stage(f"pos {pos} final norm", hf, x, om_.norms[2 * L])
        bitlinear_stage(f"pos {pos} head", L, 0, hf, lg, code)
    assert n_products == len(prompt) * (5 * L + 1)
    say(f"[info] {which}: {n_products} products exact; worst y error / tolerance {worst['y_rel']:.3f}, "
        f"worst norm rel {worst['norm_rel']:.2e}, worst SwiGLU rel {worst['swiglu_rel']:.2e}")


@pytest.mark.parametrize("which", ["model_pair", "small_pair"])
def test_decode_steps_against_oracle(which, request):
    """Trajectory smoke check on top of the stage-by-stage test: twelve
    teacher-forced steps of the seeded prompt against an oracle run that never
    sees the GPU's values.  Before the first quantised input the two agree to
    fp32 rounding; after it a value that fp32 and binary64 place on opposite
    sides of a rounding boundary may move one int8 code, so the intermediates,
    logits and caches are compared by relative norm (5e-2), and the greedy
    token must match unless the oracle's top two logits are within the
    observed logit error; the 256-d model (the fused form) and the small
    irregular one (the general form)."""
    import torch
    gm, om_ = request.getfixturevalue(which)
    d, L, ff, V, C = om_.d, om_.n_layers, om_.d_ff, om_.vocab, om_.context
    prompt = workloads.decode_model_tokens(12, V)
    gm.k_cache.zero_()
    gm.v_cache.zero_()
    kc = np.zeros((L, C, d))
    vc = np.zeros((L, C, d))
    ls = 12 * d + 3 * ff
    worst = {}
    for pos, tok in enumerate(prompt):
        say(f"[case] decode step pos={pos} token={tok}")
        st = _state(int(tok), pos)
        logits = torch.empty(V, device="cuda")
        trace = torch.full((gm.trace_floats,), float("nan"), device="cuda")
        gm.step(st, logits, trace=trace)
        torch.cuda.synchronize()
        o_logits, o_next, o_tr = om.decode_step(om_, int(tok), pos, kc, vc)
        tr = trace.cpu().numpy()
        lg = logits.cpu().numpy()
        s = st.cpu().numpy()
        # the greedy token is the argmax of the GPU's own logits, lowest index on ties
        g_next = int(np.flatnonzero(lg == lg.max())[0])
        assert s.tolist() == [g_next, pos + 1, 0, 0]
        # embedding row exact; its norm to fp32 rounding
        assert np.array_equal(tr[:d], om_.embed[tok])
        h0 = tr[d:2 * d]
        assert np.all(np.abs(h0 - o_tr[0]["h"]) <= 1e-5 * np.abs(o_tr[0]["h"]) + 1e-30)
        names = ["h", "qkv", "q", "k", "attn", "o", "x_mid", "h2", "gate", "up", "a", "down", "x_out"]
        widths = [d, 3 * d, d, d, d, d, d, d, ff, ff, ff, d, d]
        for l in range(L):
            off = d + l * ls
            ot = dict(o_tr[l])
            ot["x_mid"] = ot["x_in"] + ot["o"]
            for nm, w in zip(names, widths):
                v = tr[off:off + w]
                off += w
                e = _rel(v, ot[nm])
                worst[nm] = max(worst.get(nm, 0.0), e)
                assert e <= 5e-2, (pos, l, nm, e)
        hf = tr[d + L * ls:d + L * ls + d]
        o_hf = om.rmsnorm(o_tr[-1]["x_out"], om_.norms[2 * L])
        assert _rel(hf, o_hf) <= 5e-2
        el = _rel(lg, o_logits)
        worst["logits"] = max(worst.get("logits", 0.0), el)
        assert el <= 5e-2, (pos, el)
        if g_next != o_next:                                 # only a near-tie may differ
            top = np.sort(o_logits)[-2:]
            assert top[1] - top[0] <= 2 * np.abs(lg - o_logits).max(), (pos, g_next, o_next)
    # caches: rows 0..11 rotated keys / values as the oracle's, the rest untouched
    kg, vg = gm.k_cache.cpu().numpy(), gm.v_cache.cpu().numpy()
    n = len(prompt)
    for l in range(L):
        assert _rel(kg[l, :n], kc[l, :n]) <= 5e-2 and _rel(vg[l, :n], vc[l, :n]) <= 5e-2
    assert not kg[:, n:].any() and not vg[:, n:].any()
    say(f"[info] worst relative differences: {worst}")


def test_graph_replay_generates_like_eager_steps(model_pair):
    """One captured step, replayed: each replay reads the token and position
    the previous one left on the device, so 20 replays generate 20 tokens -
    identical (bit for bit) to 20 eager steps, with the host reading the
    results between replays."""
    import torch
    gm, om_ = model_pair
    V, C = om_.vocab, om_.context
    start = int(workloads.decode_model_tokens(1, V, seed=3)[0])

    def generate(use_graph):
        gm.k_cache.zero_()
        gm.v_cache.zero_()
        st = _state(start, 0)
        logits = torch.empty(V, device="cuda")
        toks = torch.full((C,), -1, dtype=torch.int32, device="cuda")
        seen = []
        if use_graph:
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                gm.step(st, logits, tokens=toks)             # warm-up (position 0)
            torch.cuda.current_stream().wait_stream(s)
            torch.cuda.synchronize()
            gm.k_cache.zero_()
            gm.v_cache.zero_()
            st.copy_(_state(start, 0))
            toks.fill_(-1)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                gm.step(st, logits, tokens=toks)
            torch.cuda.synchronize()                         # capture runs nothing
            for _ in range(20):
                g.replay()
                torch.cuda.synchronize()
                seen.append(logits.cpu().numpy().copy())
        else:
            for _ in range(20):
                gm.step(st, logits, tokens=toks)
                torch.cuda.synchronize()
                seen.append(logits.cpu().numpy().copy())
        return st.cpu().numpy(), toks.cpu().numpy(), seen, gm.k_cache.cpu().numpy()

    se, te, le, ke = generate(False)
    sg, tg, lg_, kg = generate(True)
    assert se.tolist()[1:] == [20, 0, 0] and sg.tolist() == se.tolist()
    assert np.array_equal(te, tg) and (te[1:21] >= 0).all() and (te[21:] == -1).all()
    assert all(np.array_equal(a, b) for a, b in zip(le, lg_))
    assert np.array_equal(ke, kg)


def test_step_edges(model_pair):
    """A position at the end of the context: nothing is computed or written,
    the state only gets LOWBIT_STEP_POSITION.  A token past the vocabulary is
    clamped to the last one (LOWBIT_STEP_TOKEN) and otherwise equal."""
    import torch
    lb = _lb()
    gm, om_ = model_pair
    V, C = om_.vocab, om_.context
    gm.k_cache.zero_()
    gm.v_cache.zero_()
    logits = torch.empty(V, device="cuda")
    st = _state(5, C)
    gm.step(st, logits)
    torch.cuda.synchronize()
    assert st.cpu().tolist() == [5, C, 0, lb.STEP_POSITION]
    assert not gm.k_cache.any() and not gm.v_cache.any()
    st = _state(V + 7, 0)
    gm.step(st, logits)
    l1 = logits.clone()
    st2 = _state(V - 1, 0)
    gm.step(st2, logits)
    torch.cuda.synchronize()
    assert st.cpu().tolist()[1:] == [1, 0, lb.STEP_TOKEN] and st2.cpu().tolist()[3] == 0
    assert torch.equal(l1, logits) and st.cpu().tolist()[0] == st2.cpu().tolist()[0]
