"""Whole decode step through the C ABI (qd_create / qd_decode_step /
qd_set_prompt / qd_generate) against the f64 oracle."""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import LOGITS_BAR, check_greedy, host, load_golden, normwise, record, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tiny():
    return synth.make_model("tiny")


@pytest.fixture(scope="module")
def tiny_ref(tiny):
    om = oracle.Model(tiny)
    toks, margins, _ = oracle.generate(om, tiny.prompt, tiny.shape.gen)
    # teacher-forced logits of the oracle's own sequence, every position
    seq = list(tiny.prompt) + list(toks[:-1])
    om2 = oracle.Model(tiny)
    logits = np.stack([om2.step(int(t), p) for p, t in enumerate(seq)])
    return toks, margins, seq, logits


def _gen(model, prompt, G):
    """qd_set_prompt + qd_generate over P+G-1 steps; returns all step argmaxes."""
    import torch
    P = len(prompt)
    out = torch.full((P + G - 1,), -1, dtype=torch.int32, device="cuda")
    model.set_prompt(prompt)
    model.generate(0, P + G - 1, tokens=out)
    return host(out)


def _teacher_forced_logits(model, seq, V):
    import torch
    lg = torch.empty((len(seq), V), dtype=torch.float32, device="cuda")
    nxt = torch.empty((len(seq),), dtype=torch.int32, device="cuda")
    for p, t in enumerate(seq):
        model.decode_step(int(t), p, logits=lg[p], next_tok=nxt[p:p + 1])
    return host(lg), host(nxt)


def _greedy_gate(got, toks, margins, label, lg=None, ref=None, P=None):
    """Every free-running greedy token equal to the oracle's; a divergence is
    accepted only at a step whose oracle margin is below the logit error
    measured there (teacher-forced logits lg against the oracle's ref, greedy
    step i at position P-1+i), when those logits are given."""
    step_err = None
    if lg is not None:
        step_err = lambda i: float(np.max(np.abs(lg[P - 1 + i] - ref[P - 1 + i])))
    n, tie = check_greedy(got, toks, margins, label, step_err)
    assert n == len(toks) or tie


@pytest.mark.parametrize("graph", [True, False])
def test_tiny_teacher_forced_logits(tiny, tiny_ref, graph):
    import token_decode_q4_amd as qd
    say(f"tiny teacher-forced logits graph={graph}")
    toks, margins, seq, ref = tiny_ref
    m = qd.Model(tiny, use_graph=graph)
    lg, nxt = _teacher_forced_logits(m, seq, tiny.shape.vocab)
    err = float(np.max(np.abs(lg - ref)))
    say(f"tiny logits max abs err {err:.3e} (scale {np.abs(ref).max():.2f})")
    assert err <= LOGITS_BAR
    assert err <= 1e-4
    # teacher-forced greedy choices equal the oracle's (f32-rounded) argmax
    P = tiny.shape.prompt_len
    ref_arg = np.argmax(ref.astype(np.float32), axis=1)
    assert np.array_equal(nxt[P - 1:], ref_arg[P - 1:])
    m.close()


def test_tiny_free_running_greedy(tiny, tiny_ref):
    import token_decode_q4_amd as qd
    toks, margins, _, _ = tiny_ref
    P, G = tiny.shape.prompt_len, tiny.shape.gen
    m = qd.Model(tiny, use_graph=True)
    got = _gen(m, tiny.prompt, G)[P - 1:]
    m.close()
    _, _, seq, ref = tiny_ref
    mt = qd.Model(tiny, use_graph=True)
    lg, _ = _teacher_forced_logits(mt, seq, tiny.shape.vocab)
    mt.close()
    _greedy_gate(got, toks, margins, "tiny", lg, ref, P)


def test_tiny_graph_equals_eager_bitwise(tiny):
    import torch
    import token_decode_q4_amd as qd
    P, G = tiny.shape.prompt_len, tiny.shape.gen
    res = []
    for graph in (True, False):
        m = qd.Model(tiny, use_graph=graph)
        toks = _gen(m, tiny.prompt, G)
        lg = torch.empty(tiny.shape.vocab, dtype=torch.float32, device="cuda")
        m.generate(P + G - 2, 1, logits_last=lg)   # recompute the last step
        res.append((toks, host(lg)))
        m.close()
    assert np.array_equal(res[0][0], res[1][0])
    assert np.array_equal(res[0][1], res[1][1])


def test_tiny_paged_equals_contiguous_bitwise(tiny):
    import token_decode_q4_amd as qd
    G = tiny.shape.gen
    a = _gen(qd.Model(tiny, paged=False), tiny.prompt, G)
    # shuffled physical blocks, more blocks than needed
    tbl = np.random.default_rng(3).permutation(8).astype(np.int32)
    mi = synth.ModelInputs(tiny.shape, tiny.embed, tiny.layers, tiny.final_norm, tiny.lm_head,
                           tiny.inv_freq, tiny.prompt, tbl)
    b = _gen(qd.Model(mi, paged=True, num_kv_blocks=8), tiny.prompt, G)
    assert np.array_equal(a, b)


def test_tiny_decode_step_rejects_out_of_range(tiny):
    import token_decode_q4_amd as qd
    m = qd.Model(tiny)
    for tok, pos, code in [(tiny.shape.vocab, 0, qd._native.QD_ERANGE), (-1, 0, qd._native.QD_ERANGE),
                           (0, tiny.shape.max_seq, qd._native.QD_ERANGE), (0, -1, qd._native.QD_ERANGE)]:
        with pytest.raises(qd.QdError) as ei:
            m.decode_step(tok, pos)
        assert ei.value.code == code
    with pytest.raises(qd.QdError):
        m.generate(tiny.shape.max_seq - 2, 3)
    m.close()


def test_tiny_step_past_written_prefix_is_refused(tiny):
    """A step may start at most one position past the written K/V prefix
    (QD_ERANGE otherwise, nothing enqueued); a step at p makes [0, p] the
    prefix, so stepping back and then skipping ahead is refused too."""
    import token_decode_q4_amd as qd
    E = qd._native.QD_ERANGE
    m = qd.Model(tiny)

    def refused(f):
        with pytest.raises(qd.QdError) as ei:
            f()
        assert ei.value.code == E

    refused(lambda: m.decode_step(0, 1))
    refused(lambda: m.generate(1, 2))
    refused(lambda: m.prefill(1, 3))
    m.set_prompt(tiny.prompt)
    m.decode_step(int(tiny.prompt[0]), 0)
    m.decode_step(int(tiny.prompt[1]), 1)
    refused(lambda: m.decode_step(0, 3))
    m.generate(2, 3)            # positions 2 .. 4
    refused(lambda: m.prefill(6, 2))
    m.prefill(5, 2)             # positions 5, 6
    m.generate(7, 1)
    m.decode_step(0, 2)         # back to position 2: the prefix is now [0, 2]
    refused(lambda: m.decode_step(0, 4))
    refused(lambda: m.generate(4, 1))
    m.decode_step(0, 3)
    m.check()
    m.close()


def _golden_run(name, layer_kernel=False, prefill=False):
    import torch
    import token_decode_q4_amd as qd
    g = load_golden(name)
    if g is None:
        pytest.skip(f"tests/golden/greedy_{name}.json not generated")
    say(f"{name}: generating inputs")
    mi = synth.make_model(name)
    assert mi.digest == g["digest"], "inputs differ from the ones the golden file was made from"
    s = mi.shape
    P, G = s.prompt_len, s.gen
    say(f"{name}: qd_create")
    say(f"{name}: qd_create (layer_kernel={layer_kernel}, prefill={prefill})")
    m = qd.Model(mi, use_graph=True, layer_kernel=layer_kernel)
    V = s.vocab
    # sample points: prefill positions and greedy steps (greedy step i is at position P-1+i)
    points = {}
    for tag in g["samples"]:
        kind, k = tag.split(":")
        pos = int(k) if kind == "prefill" else P - 1 + int(k)
        points[pos] = tag
    toks = torch.full((P + G - 1,), -1, dtype=torch.int32, device="cuda")
    lg = torch.empty(V, dtype=torch.float32, device="cuda")
    m.set_prompt(mi.prompt)
    got_logits = {}
    pos = 0
    # with prefill: positions 0 .. P-2 through qd_prefill (sampled ones as the
    # last position of a prefill call), the step at P-1 onwards as generation
    stops = sorted(set(points) | ({P - 1} if prefill else set())) + [P + G - 1]
    for stop in stops:
        if stop < pos:
            continue
        n = stop + 1 - pos if stop in points else stop - pos
        if n > 0:
            if prefill and pos + n <= P - 1:
                m.prefill(pos, n, logits_last=lg)
            else:
                m.generate(pos, n, tokens=toks[pos:pos + n], logits_last=lg)
            pos += n
            if stop in points:
                got_logits[points[stop]] = host(lg).copy()
        say(f"{name}: reached position {pos}")
    all_toks = host(toks)
    m.check()
    m.close()
    greedy = all_toks[P - 1:]

    def sample_err(tag):
        lv, smp = got_logits[tag], g["samples"][tag]
        err = float(np.max(np.abs(lv[np.array(smp["idx"])] - np.array(smp["val"]))))
        return max(err, float(np.max(np.abs(lv[np.array(smp["top_idx"])] - np.array(smp["top_val"])))))

    # a divergence is judged against the error measured at that step, which
    # exists only at the steps whose oracle logits the golden file stores
    step_err = lambda i: sample_err(f"greedy:{i}") if f"greedy:{i}" in got_logits else None
    n_eq, tie = check_greedy(greedy, g["tokens"], g["margins"], name, step_err)
    assert n_eq == len(g["tokens"]) or tie
    worst = 0.0
    for tag in got_logits:
        kind, k = tag.split(":")
        if kind == "greedy" and int(k) > n_eq:
            continue   # after an accepted near-tie the contexts differ
        err = sample_err(tag)
        worst = max(worst, err)
        say(f"{name}: logits {tag} max abs err {err:.3e}")
    record(f"{name}: {len(got_logits)} sampled steps compared, worst logit error {worst:.3e}")
    assert worst <= LOGITS_BAR
    return n_eq, worst


def test_qwen3_06b_shape_vs_golden():
    n_eq, worst = _golden_run("qwen3-0.6b")
    assert worst <= 1e-3


def test_qwen3_06b_shape_prefill_vs_golden():
    """Chunked prefill (qd_prefill) of the 512-token prompt, then greedy
    generation, against the same golden file as the sequential decode."""
    n_eq, worst = _golden_run("qwen3-0.6b", prefill=True)
    assert worst <= 1e-3


def test_qwen3_8b_shape_prefill_vs_golden():
    n_eq, worst = _golden_run("qwen3-8b", prefill=True)
    assert worst <= 5e-3


def test_qwen3_8b_shape_layer_kernel_prefill_vs_golden():
    """qd_prefill into a model that decodes with the persistent layer kernel:
    both read and write the same paged cache."""
    n_eq, worst = _golden_run("qwen3-8b", layer_kernel=True, prefill=True)
    assert worst <= 5e-3


def test_qwen3_8b_shape_vs_golden():
    n_eq, worst = _golden_run("qwen3-8b")
    # regression guard well inside the 2e-2 bar: 36 layers, rows of 12288 and
    # 2560-key softmaxes in f32 put the measured error near 2e-3
    assert worst <= 5e-3


def test_qwen3_8b_shape_layer_kernel_vs_golden():
    """The persistent layer kernel (one launch per layer, grid barriers
    between its phases) at the full shape: 36 layers, 20 attention splits,
    paged KV."""
    n_eq, worst = _golden_run("qwen3-8b", layer_kernel=True)
    assert worst <= 5e-3


def test_tiny_llama3_rope_scaling_vs_oracle(tiny):
    """The tiny model with llama3 rotary scaling (frequencies from
    qd_rope_inv_freq on the library side, from the oracle's own rule on the
    oracle side; original_max_pos 32 so that all three regimes of the rule
    occur among the 32 frequencies): teacher-forced logits and free-running
    greedy tokens."""
    import dataclasses
    import token_decode_q4_amd as qd
    s = tiny.shape
    kw = dict(scaling="llama3", factor=8.0, low_freq_factor=1.0, high_freq_factor=4.0,
              original_max_pos=32.0)
    f_lib = qd.rope_inv_freq(1e6, s.rot_dim, **kw)
    f_ref = oracle.rope_inv_freq(1e6, s.rot_dim, **kw).astype(np.float32)
    base = oracle.rope_inv_freq(1e6, s.rot_dim)
    wl = 2 * np.pi / base
    assert (wl < 8).any() and (wl > 32).any() and ((wl >= 8) & (wl <= 32)).any()
    mi_lib = dataclasses.replace(tiny, inv_freq=f_lib)
    mi_ref = dataclasses.replace(tiny, inv_freq=f_ref)
    say("tiny llama3 rotary scaling")
    om = oracle.Model(mi_ref)
    toks, margins, _ = oracle.generate(om, tiny.prompt, s.gen)
    seq = list(tiny.prompt) + list(toks[:-1])
    om2 = oracle.Model(mi_ref)
    ref = np.stack([om2.step(int(t), p) for p, t in enumerate(seq)])
    m = qd.Model(mi_lib, use_graph=True)
    lg, _ = _teacher_forced_logits(m, seq, s.vocab)
    err = float(np.max(np.abs(lg - ref)))
    say(f"tiny llama3 logits max abs err {err:.3e}")
    assert err <= 1e-4
    got = _gen(m, tiny.prompt, s.gen)[s.prompt_len - 1:]
    m.close()
    _greedy_gate(got, toks, margins, "tiny llama3", lg, ref, s.prompt_len)


@pytest.mark.parametrize("paged", [False, True])
def test_tiny_kv_fp8_vs_oracle(tiny, paged):
    """The tiny model with an fp8 e4m3 K/V cache (k_scale 0.5, v_scale 0.125)
    against the oracle storing its own K/V the same way (value / scale
    rounded to e4m3, nearest even, saturating): teacher-forced logits,
    free-running greedy tokens, and graph == eager bitwise."""
    import token_decode_q4_amd as qd
    s = tiny.shape
    ks, vs = 0.5, 0.125
    say(f"tiny fp8 KV paged={paged}")
    om = oracle.Model(tiny, kv_fp8=True, k_scale=ks, v_scale=vs)
    toks, margins, _ = oracle.generate(om, tiny.prompt, s.gen)
    seq = list(tiny.prompt) + list(toks[:-1])
    om2 = oracle.Model(tiny, kv_fp8=True, k_scale=ks, v_scale=vs)
    ref = np.stack([om2.step(int(t), p) for p, t in enumerate(seq)])
    m = qd.Model(tiny, use_graph=True, paged=paged, kv_fp8=True, k_scale=ks, v_scale=vs)
    lg, _ = _teacher_forced_logits(m, seq, s.vocab)
    err = float(np.max(np.abs(lg - ref)))
    say(f"tiny fp8 KV logits max abs err {err:.3e}")
    assert err <= LOGITS_BAR
    got = _gen(m, tiny.prompt, s.gen)[s.prompt_len - 1:]
    m.close()
    _greedy_gate(got, toks, margins, "tiny fp8 KV", lg, ref, s.prompt_len)
    me = qd.Model(tiny, use_graph=False, paged=paged, kv_fp8=True, k_scale=ks, v_scale=vs)
    lg_e, _ = _teacher_forced_logits(me, seq, s.vocab)
    me.close()
    assert np.array_equal(lg, lg_e)


@pytest.mark.parametrize("paged", [False, True])
def test_tiny_attn_out_gate_vs_oracle(paged):
    """The tiny model with an attention output gate (gate rows fused after
    q|k|v, sigmoid applied to the merged attention output): teacher-forced
    logits, free-running greedy tokens, graph == eager bitwise."""
    import token_decode_q4_amd as qd
    mi = synth.make_model("tiny", attn_out_gate=True)
    s = mi.shape
    say(f"tiny attention output gate paged={paged}")
    om = oracle.Model(mi)
    toks, margins, _ = oracle.generate(om, mi.prompt, s.gen)
    seq = list(mi.prompt) + list(toks[:-1])
    om2 = oracle.Model(mi)
    ref = np.stack([om2.step(int(t), p) for p, t in enumerate(seq)])
    m = qd.Model(mi, use_graph=True, paged=paged)
    lg, _ = _teacher_forced_logits(m, seq, s.vocab)
    err = float(np.max(np.abs(lg - ref)))
    say(f"tiny gated logits max abs err {err:.3e}")
    assert err <= 1e-4
    got = _gen(m, mi.prompt, s.gen)[s.prompt_len - 1:]
    m.close()
    _greedy_gate(got, toks, margins, "tiny gated", lg, ref, s.prompt_len)
    me = qd.Model(mi, use_graph=False, paged=paged)
    lg_e, _ = _teacher_forced_logits(me, seq, s.vocab)
    me.close()
    assert np.array_equal(lg, lg_e)


@pytest.mark.parametrize("paged,kv_fp8", [(False, False), (True, False), (False, True), (True, True)])
def test_tiny_prefill_vs_oracle(tiny, paged, kv_fp8):
    """qd_prefill of the 16-token prompt (one chunk, a quarter of its vector
    slots in use), then qd_generate from position 16: logits at the last
    prompt position against the oracle's, and the free-running greedy tokens."""
    import torch
    import token_decode_q4_amd as qd
    s = tiny.shape
    P, G = s.prompt_len, s.gen
    kw = dict(kv_fp8=True, k_scale=0.5, v_scale=0.125) if kv_fp8 else {}
    say(f"tiny prefill paged={paged} kv_fp8={kv_fp8}")
    om = oracle.Model(tiny, **kw)
    toks, margins, _ = oracle.generate(om, tiny.prompt, G)
    om2 = oracle.Model(tiny, **kw)
    for p, t in enumerate(tiny.prompt):
        ref = om2.step(int(t), p)
    m = qd.Model(tiny, use_graph=True, paged=paged, **kw)
    m.set_prompt(tiny.prompt)
    lg = torch.empty(s.vocab, dtype=torch.float32, device="cuda")
    m.prefill(0, P, logits_last=lg)
    err = float(np.max(np.abs(host(lg) - ref)))
    say(f"tiny prefill logits max abs err {err:.3e}")
    # an fp8 cache turns f32-vs-f64 differences into whole e4m3 steps where a
    # value sits near a rounding boundary, so it gets the bar of the fp8
    # decode test
    assert err <= (LOGITS_BAR if kv_fp8 else 1e-4)
    out = torch.full((G - 1,), -1, dtype=torch.int32, device="cuda")
    m.generate(P, G - 1, tokens=out)
    m.check()
    m.close()
    # the prefill's prediction at P-1 became the token at P; the generated
    # steps predict the rest
    got = np.concatenate([[int(np.argmax(host(lg)))], host(out)])
    _greedy_gate(got, toks, margins, "tiny prefill")


def test_tiny_prefill_ragged_chunks_vs_oracle():
    """The tiny decoder with a 160-position cache: 100 teacher-forced
    positions prefilled as C + 5 and 95 - C positions (C = qd.prefill_chunk():
    a full chunk, a ragged one, then a call continuing the cache in a ragged
    chunk), logits at the last position of each call against the oracle's,
    then generation of the remaining greedy tokens."""
    import dataclasses
    import torch
    import token_decode_q4_amd as qd
    shape = dataclasses.replace(synth.MODELS["tiny"], name="tiny-long", max_seq=160, gen=145)
    mi = synth.make_model(shape)
    P, G = shape.prompt_len, shape.gen
    toks, margins, _ = oracle.generate(oracle.Model(mi), mi.prompt, G)
    seq = list(mi.prompt) + list(toks[:-1])
    om = oracle.Model(mi)
    ref = np.stack([om.step(int(t), p) for p, t in enumerate(seq)])
    n = 100
    n1 = qd.prefill_chunk() + 5
    assert n1 < n <= shape.max_seq - 1
    say("tiny prefill ragged chunks")
    m = qd.Model(mi, use_graph=True)
    m.set_prompt(seq[:n])
    lg = torch.empty(shape.vocab, dtype=torch.float32, device="cuda")
    m.prefill(0, n1, logits_last=lg)
    e1 = float(np.max(np.abs(host(lg) - ref[n1 - 1])))
    m.prefill(n1, n - n1, logits_last=lg)
    e2 = float(np.max(np.abs(host(lg) - ref[n - 1])))
    say(f"tiny ragged prefill logits max abs err {e1:.3e} {e2:.3e}")
    assert max(e1, e2) <= 1e-4
    rest = shape.max_seq - 1 - n
    out = torch.full((rest,), -1, dtype=torch.int32, device="cuda")
    m.generate(n, rest, tokens=out)
    m.check()
    m.close()
    # the step at position p predicts greedy token p - (P - 1); the first
    # compared token is the prefill's prediction at n - 1
    i0 = n - P
    got = np.concatenate([[int(np.argmax(host(lg)))], host(out)])
    _greedy_gate(got, toks[i0:i0 + len(got)], margins[i0:i0 + len(got)], "tiny ragged prefill")


def test_tiny_long_prefill_vs_oracle():
    """qd_prefill over 4096 positions of the tiny decoder on a paged cache, in
    two calls (0 .. 2047, 2048 .. 4095): the chunk attention's splits grow with
    the context (up to 64 per chunk), so the split merge takes every one of
    its round sizes (U = 2 .. 32 splits per thread group); logits at the last
    position of each call against the oracle's teacher-forced ones (<= 1e-4),
    and the prediction at 4095."""
    import dataclasses
    import torch
    import token_decode_q4_amd as qd
    shape = dataclasses.replace(synth.MODELS["tiny"], name="tiny-4k", max_seq=4160, prompt_len=4096, gen=8)
    mi = synth.make_model(shape)
    n, half = 4096, 2048
    om = oracle.Model(mi)
    ref = {}
    for p in range(n):
        lg_o = om.step(int(mi.prompt[p]), p)
        if p in (half - 1, n - 1):
            ref[p] = lg_o
    say("tiny long prefill")
    nblk = (shape.max_seq + 15) // 16 + 3
    tbl = np.random.default_rng(17).permutation(nblk).astype(np.int32)
    src = synth.ModelInputs(mi.shape, mi.embed, mi.layers, mi.final_norm, mi.lm_head, mi.inv_freq,
                            mi.prompt, tbl, mi.digest)
    m = qd.Model(src, use_graph=True, paged=True, num_kv_blocks=nblk)
    m.set_prompt(mi.prompt)
    lg = torch.empty(shape.vocab, dtype=torch.float32, device="cuda")
    m.prefill(0, half, logits_last=lg)
    e1 = float(np.max(np.abs(host(lg) - ref[half - 1])))
    m.prefill(half, n - half, logits_last=lg)
    got = host(lg)
    e2 = float(np.max(np.abs(got - ref[n - 1])))
    m.check()
    m.close()
    say(f"tiny long prefill logits max abs err {e1:.3e} (position {half - 1}), {e2:.3e} (position {n - 1})")
    assert max(e1, e2) <= 1e-4
    r = ref[n - 1].astype(np.float32)
    top2 = np.sort(r)[-2:]
    assert int(np.argmax(got)) == int(np.argmax(r)) or top2[1] - top2[0] < e2


def test_tiny_prefill_rejects(tiny):
    import token_decode_q4_amd as qd
    m = qd.Model(tiny)
    for pos0, n in [(0, 0), (-1, 4), (tiny.shape.max_seq, 1), (tiny.shape.max_seq - 3, 4)]:
        with pytest.raises(qd.QdError) as ei:
            m.prefill(pos0, n)
        assert ei.value.code == qd._native.QD_ERANGE
    m.close()


@pytest.mark.parametrize("paged", [False, True])
def test_tiny_gated_prefill_vs_oracle(paged):
    """qd_prefill of a model with the attention output gate: logits at the
    last prompt position against the oracle, then greedy generation."""
    import torch
    import token_decode_q4_amd as qd
    mi = synth.make_model("tiny", attn_out_gate=True)
    s = mi.shape
    P, G = s.prompt_len, s.gen
    say(f"tiny gated prefill paged={paged}")
    toks, margins, _ = oracle.generate(oracle.Model(mi), mi.prompt, G)
    om = oracle.Model(mi)
    for p, t in enumerate(mi.prompt):
        ref = om.step(int(t), p)
    m = qd.Model(mi, use_graph=True, paged=paged)
    m.set_prompt(mi.prompt)
    lg = torch.empty(s.vocab, dtype=torch.float32, device="cuda")
    m.prefill(0, P, logits_last=lg)
    err = float(np.max(np.abs(host(lg) - ref)))
    say(f"tiny gated prefill logits max abs err {err:.3e}")
    assert err <= 1e-4
    out = torch.full((G - 1,), -1, dtype=torch.int32, device="cuda")
    m.generate(P, G - 1, tokens=out)
    m.check()
    m.close()
    got = np.concatenate([[int(np.argmax(host(lg)))], host(out)])
    _greedy_gate(got, toks, margins, "tiny gated prefill")


# Regression guards on the variants' teacher-forced logits (max abs), far
# inside the c14 parity bar of 2e-2 and a few times above each model's
# measured f32 error: the tiny family's is 2.5e-5 .. 5e-5; tiny-odd, another
# random draw, sits at 1.4e-4 on both the decode and the batched paths (the
# tiny weights with only the vocabulary cut to 1000 show the same level, so
# it is the draw's conditioning, not its sizes).
_VARIANT_GUARD = {"tiny-odd": 5e-4}


def _variant_ref(name):
    mi = synth.make_model(name)
    om = oracle.Model(mi)
    toks, margins, _ = oracle.generate(om, mi.prompt, mi.shape.gen)
    seq = list(mi.prompt) + list(toks[:-1])
    om2 = oracle.Model(mi)
    ref = np.stack([om2.step(int(t), p) for p, t in enumerate(seq)])
    return mi, toks, margins, seq, ref


def _paged_inputs(mi, nblocks=8):
    """The same model with a shuffled physical block table (more blocks than
    max_seq needs)."""
    tbl = np.random.default_rng(5).permutation(nblocks).astype(np.int32)
    return synth.ModelInputs(mi.shape, mi.embed, mi.layers, mi.final_norm, mi.lm_head, mi.inv_freq,
                             mi.prompt, tbl, mi.digest)


@pytest.mark.parametrize("name,paged", [("tiny-rot32", False), ("tiny-rot32", True),
                                        ("tiny-untied", False), ("tiny-untied", True),
                                        ("tiny-odd", False), ("tiny-odd", True), ("tiny-gq8", True),
                                        ("tiny-mha", False)])
def test_tiny_variant_decode_vs_oracle(name, paged):
    """Partial rotary (rot_dim 32 of head_dim 64), an untied LM head, sizes
    that are not multiples of 256 (hidden 288, SwiGLU 800, vocab 1000) and
    GQA groups of 8 and 1 through the decode step: teacher-forced logits of every position (<= 1e-4 abs) and
    the teacher-forced argmax, free-running greedy tokens, graph == eager."""
    import token_decode_q4_amd as qd
    mi, toks, margins, seq, ref = _variant_ref(name)
    s = mi.shape
    P = s.prompt_len
    say(f"{name} decode paged={paged}")
    src = _paged_inputs(mi) if paged else mi
    kw = dict(paged=True, num_kv_blocks=8) if paged else {}
    m = qd.Model(src, use_graph=True, **kw)
    lg, nxt = _teacher_forced_logits(m, seq, s.vocab)
    err = float(np.max(np.abs(lg - ref)))
    say(f"{name} paged={paged}: logits max abs err {err:.3e} over {len(seq)} positions")
    assert err <= _VARIANT_GUARD.get(name, 1e-4)
    assert np.array_equal(nxt[P - 1:], np.argmax(ref.astype(np.float32), axis=1)[P - 1:])
    got = _gen(m, mi.prompt, s.gen)[P - 1:]
    m.close()
    _greedy_gate(got, toks, margins, f"{name} paged={paged}", lg, ref, P)
    me = qd.Model(src, use_graph=False, **kw)
    lg_e, _ = _teacher_forced_logits(me, seq, s.vocab)
    me.close()
    assert np.array_equal(lg, lg_e)


@pytest.mark.parametrize("name,paged", [("tiny-rot32", False), ("tiny-rot32", True),
                                        ("tiny-untied", False), ("tiny-odd", False), ("tiny-odd", True),
                                        ("tiny-gq8", False), ("tiny-gq8", True), ("tiny-mha", False),
                                        ("tiny-mha", True)])
def test_tiny_variant_prefill_vs_oracle(name, paged):
    """qd_prefill (one chunk on the matrix-core products) of the variant's prompt:
    logits at the last prompt position (<= 1e-4), then greedy generation
    against the oracle's tokens."""
    import torch
    import token_decode_q4_amd as qd
    mi, toks, margins, seq, ref = _variant_ref(name)
    s = mi.shape
    P, G = s.prompt_len, s.gen
    say(f"{name} prefill paged={paged}")
    src = _paged_inputs(mi) if paged else mi
    kw = dict(paged=True, num_kv_blocks=8) if paged else {}
    m = qd.Model(src, use_graph=True, **kw)
    m.set_prompt(mi.prompt)
    lg = torch.empty(s.vocab, dtype=torch.float32, device="cuda")
    m.prefill(0, P, logits_last=lg)
    err = float(np.max(np.abs(host(lg) - ref[P - 1])))
    say(f"{name} prefill paged={paged}: logits max abs err {err:.3e}")
    assert err <= _VARIANT_GUARD.get(name, 1e-4)
    out = torch.full((G - 1,), -1, dtype=torch.int32, device="cuda")
    m.generate(P, G - 1, tokens=out)
    m.check()
    m.close()
    got = np.concatenate([[int(np.argmax(host(lg)))], host(out)])
    _greedy_gate(got, toks, margins, f"{name} prefill paged={paged}")


def test_tiny_prefill_large_activations_vs_oracle():
    """The tiny model with every post-attention norm weight times 4096: the
    SwiGLU outputs reach ~1e6, beyond f16 range, so the prefill's matrix-core
    products must scale each position's activations before splitting them into
    f16 halves.  Prefill logits at the last prompt position and decode-step
    logits against the oracle (normwise 1e-4)."""
    import dataclasses
    import torch
    import token_decode_q4_amd as qd
    tiny = synth.make_model("tiny")
    mi = dataclasses.replace(tiny, layers=[dataclasses.replace(L, ffn_norm=(L.ffn_norm * np.float32(4096)))
                                           for L in tiny.layers])
    s = mi.shape
    P = s.prompt_len
    say("tiny prefill with large activations")
    om = oracle.Model(mi)
    for p, t in enumerate(mi.prompt):
        ref = om.step(int(t), p)
    m = qd.Model(mi, use_graph=True)
    m.set_prompt(mi.prompt)
    lg = torch.empty(s.vocab, dtype=torch.float32, device="cuda")
    m.prefill(0, P, logits_last=lg)
    got = host(lg)
    m.close()
    md = qd.Model(mi, use_graph=True)
    md.set_prompt(mi.prompt)
    ld = torch.empty(s.vocab, dtype=torch.float32, device="cuda")
    md.generate(0, P, logits_last=ld)
    dec = host(ld)
    md.close()
    e_pf, e_dec = normwise(got, ref), normwise(dec, ref)
    say(f"large activations: prefill normwise err {e_pf:.2e}, decode {e_dec:.2e}")
    assert np.all(np.isfinite(got))
    assert e_pf <= 1e-4 and e_dec <= 1e-4
