"""The persistent layer kernel (qd_config.layer_kernel = 1: one launch per
layer, device-wide barriers between its phases) through the C ABI, against the
f64 oracle and against the per-layer kernels."""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import LOGITS_BAR, check_greedy, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lk():
    import torch
    torch.cuda.set_device(0)   # the HIP runtime comes up before the oracle's threads
    say("layerk: generating inputs")
    return synth.make_model("layerk")


@pytest.fixture(scope="module")
def lk_ref(lk):
    """Oracle greedy sequence and its logits at every position (prompt fed at
    0..P-1, then each greedy token at the next position)."""
    say("layerk: oracle")
    P, G = lk.shape.prompt_len, lk.shape.gen
    toks, margins, _ = oracle.generate(oracle.Model(lk), lk.prompt, G)
    seq = list(lk.prompt) + list(toks[:-1])
    om = oracle.Model(lk)
    logits = np.stack([om.step(int(t), p) for p, t in enumerate(seq)])
    return toks, margins, seq, logits


def _teacher_forced(model, seq, V):
    import torch
    lg = torch.empty((len(seq), V), dtype=torch.float32, device="cuda")
    nxt = torch.empty((len(seq),), dtype=torch.int32, device="cuda")
    for p, t in enumerate(seq):
        model.decode_step(int(t), p, logits=lg[p], next_tok=nxt[p:p + 1])
    return host(lg), host(nxt)


@pytest.mark.parametrize("paged", [True, False])
def test_layer_kernel_teacher_forced_logits(lk, lk_ref, paged):
    import token_decode_q4_amd as qd
    say(f"layerk teacher-forced logits, layer kernel, paged={paged}")
    toks, margins, seq, ref = lk_ref
    m = qd.Model(lk, use_graph=True, paged=paged, layer_kernel=True)
    lg, nxt = _teacher_forced(m, seq, lk.shape.vocab)
    m.close()
    err = float(np.max(np.abs(lg - ref)))
    say(f"layerk logits max abs err {err:.3e} (scale {np.abs(ref).max():.2f})")
    assert np.all(np.isfinite(lg))
    assert err <= LOGITS_BAR
    assert err <= 2e-3
    P = lk.shape.prompt_len
    ref_arg = np.argmax(ref.astype(np.float32), axis=1)
    assert np.array_equal(nxt[P - 1:], ref_arg[P - 1:])


def test_layer_kernel_matches_per_layer_kernels(lk, lk_ref):
    """Same step, two kernel plans: equal up to f32 rounding order (the RMS
    partial sums are grouped by a different grid)."""
    import token_decode_q4_amd as qd
    _, _, seq, ref = lk_ref
    out = []
    for layer_kernel in (False, True):
        m = qd.Model(lk, use_graph=True, layer_kernel=layer_kernel)
        out.append(_teacher_forced(m, seq, lk.shape.vocab)[0])
        m.close()
    d = float(np.max(np.abs(out[0] - out[1])))
    say(f"layerk: layer kernel vs per-layer kernels max abs diff {d:.3e}")
    assert d <= 1e-3


def test_layer_kernel_free_running_greedy(lk, lk_ref):
    import torch
    import token_decode_q4_amd as qd
    toks, margins, _, _ = lk_ref
    P, G = lk.shape.prompt_len, lk.shape.gen
    m = qd.Model(lk, use_graph=True, layer_kernel=True)
    out = torch.full((P + G - 1,), -1, dtype=torch.int32, device="cuda")
    m.set_prompt(lk.prompt)
    m.generate(0, P + G - 1, tokens=out)
    got = host(out)[P - 1:]
    m.close()
    assert check_greedy(got, toks, margins, "layerk") == (G, False)


def test_layer_kernel_graph_equals_eager_bitwise(lk):
    import torch
    import token_decode_q4_amd as qd
    P, G = lk.shape.prompt_len, lk.shape.gen
    res = []
    for graph in (True, False):
        m = qd.Model(lk, use_graph=graph, layer_kernel=True)
        out = torch.full((P + G - 1,), -1, dtype=torch.int32, device="cuda")
        m.set_prompt(lk.prompt)
        m.generate(0, P + G - 1, tokens=out)
        lg = torch.empty(lk.shape.vocab, dtype=torch.float32, device="cuda")
        m.generate(P + G - 2, 1, logits_last=lg)
        res.append((host(out), host(lg)))
        m.close()
    assert np.array_equal(res[0][0], res[1][0])
    assert np.array_equal(res[0][1], res[1][1])


def test_layer_kernel_barrier_timeout_is_reported(lk, monkeypatch):
    """A barrier that gives up waiting (forced from the host with a spin bound
    of 0 polls; every wait still ends) is reported by qd_check, and a model
    with the normal bound reports nothing."""
    import token_decode_q4_amd as qd
    P = lk.shape.prompt_len
    monkeypatch.setenv("QD_LAYER_KERNEL_SPIN_LIMIT", "0")
    m = qd.Model(lk, use_graph=True, layer_kernel=True)
    monkeypatch.delenv("QD_LAYER_KERNEL_SPIN_LIMIT")
    m.set_prompt(lk.prompt)
    m.generate(0, 8)
    with pytest.raises(qd.QdError) as ei:
        m.check()
    assert ei.value.code == qd._native.QD_EHIP and "barrier" in str(ei.value)
    m.check()   # cleared
    m.close()
    m = qd.Model(lk, use_graph=True, layer_kernel=True)
    m.set_prompt(lk.prompt)
    m.generate(0, P - 1)
    m.check()
    m.close()
