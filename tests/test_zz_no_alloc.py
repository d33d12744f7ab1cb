"""The allocation-free decode step (lowbit_decode_step_noalloc) against the
decode step with a caller workspace (lowbit_decode_step), through the C ABI.

Two calls in a row of each entry point, the second on a smaller model: the
256-d 6-layer model (the fused form, 4096-entry vocabulary), then a 64-d
2-layer model with an irregular FFN width (the general form).  Both run the
same kernels on the same inputs, so logits, the state, the key/value caches,
the generated token and every traced intermediate and code record must be
identical bit for bit; the second call also shows that the static workspace
keeping the first call's contents changes nothing.  Host-side checks (the
workspace bound, NULL work accepted) run without a GPU in test_abi_cpu.py.
"""
import numpy as np
import pytest

import workloads
from tests.gpu_common import say
from tests.test_gpu_model import _build_pair, _latent, _state, CFG

pytestmark = pytest.mark.gpu


def _run(gm, vocab, tok, pos, noalloc):
    import torch
    gm.k_cache.zero_()
    gm.v_cache.zero_()
    st = _state(tok, pos)
    logits = torch.full((vocab,), float("nan"), device="cuda")
    toks = torch.full((gm.model.context,), -1, dtype=torch.int32, device="cuda")
    trace = torch.full((gm.trace_floats,), float("nan"), device="cuda")
    if noalloc:
        gm.work.fill_(0xA5)            # the caller workspace is not what the no-alloc call reads
    gm.step(st, logits, tokens=toks, trace=trace, noalloc=noalloc)
    torch.cuda.synchronize()
    return (st.cpu().numpy(), logits.cpu().numpy(), toks.cpu().numpy(), trace.cpu().numpy(),
            gm.k_cache.cpu().numpy(), gm.v_cache.cpu().numpy())


def _same(a, b):
    return all(np.array_equal(x.view(np.uint8), y.view(np.uint8)) for x, y in zip(a, b))


def test_noalloc_step_equals_workspace_step():
    import torch
    big = _build_pair(*(CFG[k] for k in ("d", "layers", "heads", "d_ff", "vocab", "context")), _latent)
    small = _build_pair(64, 2, 1, 98, 300, 16,
                        lambda layer, slot, n, k: workloads.random_case(1200 + 7 * layer + slot, n, k, 1)[0])
    for name, (gm, om_), tok, pos in (("256-d model", big, 17, 0), ("64-d model", small, 5, 3)):
        say(f"[case] noalloc decode step: {name} token={tok} pos={pos}")
        ref = _run(gm, om_.vocab, tok, pos, noalloc=False)
        got = _run(gm, om_.vocab, tok, pos, noalloc=True)
        assert ref[0].tolist()[1:] == [pos + 1, 0, 0]
        assert np.isfinite(ref[1]).all()
        assert _same(ref, got), name
    # the small model again without the trace: the path the timed decode takes
    gm, om_ = small
    gm.k_cache.zero_()
    st_a, st_b = _state(5, 0), _state(5, 0)
    la = torch.empty(om_.vocab, device="cuda")
    lb_ = torch.empty(om_.vocab, device="cuda")
    gm.step(st_a, la)
    ka = gm.k_cache.clone()
    gm.k_cache.zero_()
    gm.step(st_b, lb_, noalloc=True)
    torch.cuda.synchronize()
    assert torch.equal(la, lb_) and torch.equal(st_a, st_b) and torch.equal(ka, gm.k_cache)
