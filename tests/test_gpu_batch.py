"""Batched decode (qd_create_batch / qd_generate_batch / qd_decode_step_batch):
B sequences stepped together, each against the f64 oracle run on its own."""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import LOGITS_BAR, check_greedy, host, load_golden, record, say

pytestmark = pytest.mark.gpu


def _prompts(mi, B, lo, hi, seed=77):
    """B seeded prompts of ragged lengths in [lo, hi]."""
    rng = np.random.default_rng(seed)
    return [rng.integers(0, mi.shape.vocab, size=int(rng.integers(lo, hi + 1))).astype(np.int32)
            for _ in range(B)]


def _oracle_runs(mi, prompts, S, **kw):
    """Per sequence: greedy tokens and margins of S lockstep steps (positions
    0 .. S-1, the prompt forced), the oracle's sequence and its teacher-forced
    logits."""
    out = []
    for pr in prompts:
        G = S - len(pr) + 1
        toks, margins, _ = oracle.generate(oracle.Model(mi, **kw), pr, G)
        seq = list(pr) + list(toks[:-1])
        om = oracle.Model(mi, **kw)
        ref = np.stack([om.step(int(t), p) for p, t in enumerate(seq)])
        out.append((toks, margins, seq, ref))
    return out


def _paged_table(B, max_seq, seed=9, spare=3):
    need = (max_seq + 15) // 16
    perm = np.random.default_rng(seed).permutation(B * need + spare).astype(np.int32)
    return perm[:B * need].reshape(B, need), B * need + spare


def _batch_model(mi, B, paged, **kw):
    import token_decode_q4_amd as qd
    if paged:
        tbl, nblk = _paged_table(B, mi.shape.max_seq)
        return qd.Model(mi, batch=B, paged=True, block_table=tbl, num_kv_blocks=nblk, **kw)
    return qd.Model(mi, batch=B, paged=False, **kw)


def _run_lockstep(m, prompts, S):
    """Prompts set per sequence, then S steps of every sequence at once."""
    import torch
    B = len(prompts)
    for b, pr in enumerate(prompts):
        m.set_prompt_seq(b, pr)
    toks = torch.full((B, S), -1, dtype=torch.int32, device="cuda")
    m.generate_batch([0] * B, S, tokens=toks)
    m.check()
    return host(toks)


def _teacher_forced_batch(m, runs, S, V):
    """Logits [B][S][V] of qd_decode_step_batch along each oracle sequence."""
    import torch
    B = len(runs)
    lg = np.zeros((B, S, V), np.float32)
    dl = torch.empty((B, V), dtype=torch.float32, device="cuda")
    for p in range(S):
        m.decode_step_batch([runs[b][2][p] for b in range(B)], [p] * B, logits=dl)
        lg[:, p] = host(dl)
    m.check()
    return lg


def _compare(got, prompts, runs, label, lg=None):
    for b, (pr, (toks, margins, seq, ref)) in enumerate(zip(prompts, runs)):
        P = len(pr)
        step_err = None
        if lg is not None:
            step_err = lambda i, b=b, ref=ref, P=P: float(np.max(np.abs(lg[b][P - 1 + i] - ref[P - 1 + i])))
        n, tie = check_greedy(got[b, P - 1:], toks, margins, f"{label} seq {b} (prompt {P})", step_err)
        assert n == len(toks) or tie


@pytest.fixture(scope="module")
def tiny():
    return synth.make_model("tiny")


TINY_S = 47   # steps: positions 0 .. 46 of max_seq 48


@pytest.fixture(scope="module")
def tiny_runs(tiny):
    prompts = _prompts(tiny, 16, 8, 16)
    return prompts, _oracle_runs(tiny, prompts, TINY_S)


@pytest.mark.parametrize("B", [2, 3, 4, 6, 8, 11, 16])
@pytest.mark.parametrize("paged", [False, True])
def test_tiny_batch_greedy_vs_oracle(tiny, tiny_runs, B, paged):
    """Each of B sequences (ragged prompts of 8 .. 16 tokens, the rest greedy)
    generates the oracle's greedy tokens.  The widths include ones that fill
    no 4-vector slot group (3, 11) and both sides of the attention's chunk
    merge (from 8)."""
    prompts, runs = tiny_runs
    say(f"tiny batch B={B} paged={paged}")
    m = _batch_model(tiny, B, paged)
    got = _run_lockstep(m, prompts[:B], TINY_S)
    m.close()
    _compare(got, prompts[:B], runs[:B], f"tiny B={B} paged={paged}")


@pytest.mark.parametrize("B", [4, 11, 16])
def test_tiny_batch_teacher_forced_logits(tiny, tiny_runs, B):
    """qd_decode_step_batch along each oracle sequence: every position's logits
    of every sequence within 1e-3 of the oracle's, and the step's argmax equal
    to the oracle's f32-rounded argmax; graph and eager launches bitwise equal."""
    import torch
    import token_decode_q4_amd as qd
    prompts, runs = tiny_runs
    V = tiny.shape.vocab
    res = []
    for graph in (True, False):
        m = qd.Model(tiny, batch=B, paged=False, use_graph=graph)
        lg = np.zeros((B, TINY_S, V), np.float32)
        nxt = np.zeros((B, TINY_S), np.int32)
        dl = torch.empty((B, V), dtype=torch.float32, device="cuda")
        dn = torch.empty(B, dtype=torch.int32, device="cuda")
        for p in range(TINY_S):
            m.decode_step_batch([runs[b][2][p] for b in range(B)], [p] * B, logits=dl, next_tok=dn)
            lg[:, p] = host(dl)
            nxt[:, p] = host(dn)
        m.check()
        m.close()
        res.append((lg, nxt))
    lg, nxt = res[0]
    assert np.array_equal(lg, res[1][0]) and np.array_equal(nxt, res[1][1])
    worst = 0.0
    for b in range(B):
        ref = runs[b][3]
        worst = max(worst, float(np.max(np.abs(lg[b] - ref))))
        P = len(prompts[b])
        assert np.array_equal(nxt[b, P - 1:], np.argmax(ref.astype(np.float32), axis=1)[P - 1:])
    record(f"tiny batch B={B}: teacher-forced logits of {B} x {TINY_S} steps, max abs err {worst:.3e}")
    # regression guard far inside the 2e-2 bar: the batched step rounds the
    # normalised activation to f32 before the product (the one-sequence step
    # scales the product instead) and its GEMVs sum in other orders; from 6
    # sequences x enters the matrix cores as an f16 pair (about 22 bits)
    assert worst <= 1e-3


@pytest.mark.parametrize("B,paged", [(4, False), (16, True)])
def test_tiny_odd_batch_vs_oracle(B, paged):
    """A model at sizes that are not multiples of 256 (hidden 288, SwiGLU 800,
    vocab 1000): the products' rows hold 9 and 25 q4_0 blocks (scales loaded
    one by one, a ragged last chunk) and the LM head ends in a partial row
    tile.  Teacher-forced logits of every sequence within 1e-3 of the oracle,
    then each sequence's greedy tokens."""
    mi = synth.make_model("tiny-odd")
    prompts = _prompts(mi, B, 8, 16, seed=79)
    runs = _oracle_runs(mi, prompts, TINY_S)
    say(f"tiny-odd batch B={B} paged={paged}")
    m = _batch_model(mi, B, paged)
    lg = _teacher_forced_batch(m, runs, TINY_S, mi.shape.vocab)
    m.close()
    worst = max(float(np.max(np.abs(lg[b] - runs[b][3]))) for b in range(B))
    record(f"tiny-odd batch B={B}: teacher-forced logits max abs err {worst:.3e}")
    assert worst <= 1e-3
    m = _batch_model(mi, B, paged)
    got = _run_lockstep(m, prompts, TINY_S)
    m.close()
    _compare(got, prompts, runs, f"tiny-odd B={B} paged={paged}", lg)


@pytest.mark.parametrize("name,B,paged", [("tiny-gq8", 16, True), ("tiny-mha", 16, False), ("tiny-mha", 4, True)])
def test_tiny_group_batch_vs_oracle(name, B, paged):
    """GQA groups of 8 (the attention's chunk merge writing the o product's
    input for one kv head) and 1 (head_dim 64: the separate split, whatever
    B) in the batched step: teacher-forced logits of every sequence within
    1e-3 of the oracle, then each sequence's greedy tokens."""
    mi = synth.make_model(name)
    prompts = _prompts(mi, B, 8, 16, seed=83)
    runs = _oracle_runs(mi, prompts, TINY_S)
    say(f"{name} batch B={B} paged={paged}")
    m = _batch_model(mi, B, paged)
    lg = _teacher_forced_batch(m, runs, TINY_S, mi.shape.vocab)
    m.close()
    worst = max(float(np.max(np.abs(lg[b] - runs[b][3]))) for b in range(B))
    record(f"{name} batch B={B}: teacher-forced logits max abs err {worst:.3e}")
    assert worst <= 1e-3
    m = _batch_model(mi, B, paged)
    got = _run_lockstep(m, prompts, TINY_S)
    m.close()
    _compare(got, prompts, runs, f"{name} B={B} paged={paged}", lg)


def test_tiny_gq8_long_batch_vs_oracle():
    """8 sequences of the GQA-8 tiny model (one kv head) with a 640-position
    cache and prompts of 560 .. 600 tokens: the attention takes ~20 key splits
    per sequence, so the chunk merge that writes the o product's input runs
    its 32-split load round.  Teacher-forced logits of every step and sequence
    within 1e-3 of the oracle, then each sequence's greedy tokens."""
    import dataclasses
    shape = dataclasses.replace(synth.MODELS["tiny-gq8"], name="tiny-gq8-640", max_seq=640)
    mi = synth.make_model(shape)
    B, S = 8, 620
    prompts = _prompts(mi, B, 560, 600, seed=89)
    runs = _oracle_runs(mi, prompts, S)
    say(f"tiny-gq8 long batch B={B}")
    m = _batch_model(mi, B, True)
    lg = _teacher_forced_batch(m, runs, S, mi.shape.vocab)
    m.close()
    worst = max(float(np.max(np.abs(lg[b] - runs[b][3]))) for b in range(B))
    record(f"tiny-gq8 long batch B={B}: teacher-forced logits of {B} x {S} steps, max abs err {worst:.3e}")
    assert worst <= 1e-3
    m = _batch_model(mi, B, True)
    got = _run_lockstep(m, prompts, S)
    m.close()
    _compare(got, prompts, runs, f"tiny-gq8 long B={B}", lg)


def test_tiny_batch_kv_fp8_vs_oracle(tiny):
    """fp8 e4m3 K/V caches in the batched step (k_scale 0.5, v_scale 0.125)."""
    B = 4
    prompts = _prompts(tiny, B, 8, 16, seed=78)
    kw = dict(kv_fp8=True, k_scale=0.5, v_scale=0.125)
    runs = _oracle_runs(tiny, prompts, TINY_S, **kw)
    m = _batch_model(tiny, B, True, **kw)
    got = _run_lockstep(m, prompts, TINY_S)
    m.close()
    _compare(got, prompts, runs, "tiny B=4 fp8")


def test_tiny_batch_refusals(tiny):
    import token_decode_q4_amd as qd
    E, R = qd._native.QD_EINVAL, qd._native.QD_ERANGE
    m = qd.Model(tiny, batch=4, paged=False)

    def code(f):
        with pytest.raises(qd.QdError) as ei:
            f()
        return ei.value.code

    assert code(lambda: m.decode_step(0, 0)) == E          # one-sequence entry points
    assert code(lambda: m.generate(0, 1)) == E
    assert code(lambda: m.prefill(0, 1)) == E
    assert code(lambda: m.set_prompt_seq(4, [1])) == E     # no such sequence
    assert code(lambda: m.generate_batch([0, 0, 1, 0], 2)) == R   # past the written prefix
    m.generate_batch([0, 0, 0, 0], 3)
    assert code(lambda: m.generate_batch([3, 3, 3, 47], 2)) == R  # beyond max_seq
    assert code(lambda: m.decode_step_batch([0, 0, 0, 0], [3, 3, 3, 5])) == R
    m.decode_step_batch([0, 0, 0, 0], [3, 3, 3, 3])
    m.check()
    m.close()
    one = qd.Model(tiny)
    assert code(lambda: one.generate_batch([0], 1)) == E
    one.close()
    with pytest.raises(qd.QdError) as ei:
        qd.Model(tiny, batch=17)
    assert ei.value.code == E


@pytest.fixture(scope="module")
def small():
    return synth.make_model("qwen3-0.6b")


SMALL_S = 32


@pytest.fixture(scope="module")
def small_runs(small):
    say("qwen3-0.6b batch: oracle runs of 16 sequences")
    prompts = _prompts(small, 16, 16, 24, seed=79)
    return prompts, _oracle_runs(small, prompts, SMALL_S)


@pytest.mark.parametrize("B", [2, 4, 8, 11, 16])
def test_qwen3_06b_shape_batch_vs_oracle(small, small_runs, B):
    """The Qwen3-0.6B shape (28 layers, vocabulary 151936) in batches of 2 to
    16 sequences with ragged prompts of 16 .. 24 tokens: every sequence's greedy
    tokens equal the oracle's."""
    import token_decode_q4_amd as qd
    prompts, runs = small_runs
    say(f"qwen3-0.6b batch B={B}")
    m = qd.Model(small, batch=B, paged=False, max_seq=SMALL_S + 1)
    got = _run_lockstep(m, prompts[:B], SMALL_S)
    # teacher-forced logits along each oracle sequence: the logit error the
    # greedy gate measures a near-tie against
    lg = _teacher_forced_batch(m, runs[:B], SMALL_S, small.shape.vocab)
    m.close()
    worst = max(float(np.max(np.abs(lg[b] - runs[b][3]))) for b in range(B))
    record(f"qwen3-0.6b B={B}: teacher-forced logits of {B} x {SMALL_S} steps, max abs err {worst:.3e}")
    assert worst <= 2e-2
    _compare(got, prompts[:B], runs[:B], f"qwen3-0.6b B={B}", lg)


@pytest.mark.parametrize("B", [4, 16])
def test_qwen3_8b_shape_batch_vs_golden(B):
    """The batched step at the benchmarked size: 4 and 16 sequences of the
    Qwen3-8B shape (the attention output split by its own kernel, and by the
    attention's chunk merge), each on its own paged cache (a shuffled table per sequence) and
    holding the 8B golden file's prompt and greedy tokens as forced tokens,
    stepped together through positions 0 .. P+G-2.  The contexts are then the
    oracle's, so at every greedy position every sequence's argmax must be the
    oracle's greedy token, and at the golden file's sampled positions every
    sequence's logits must be within the logits bar of the oracle's."""
    import torch
    import token_decode_q4_amd as qd
    g = load_golden("qwen3-8b")
    if g is None:
        pytest.skip("tests/golden/greedy_qwen3-8b.json not generated")
    say("qwen3-8b batch: generating inputs")
    mi = synth.make_model("qwen3-8b")
    assert mi.digest == g["digest"], "inputs differ from the ones the golden file was made from"
    s = mi.shape
    P, G, V = s.prompt_len, s.gen, s.vocab
    stream = np.concatenate([mi.prompt, np.asarray(g["tokens"][:G - 1], dtype=np.int32)]).astype(np.int32)
    tbl, nblk = _paged_table(B, s.max_seq, seed=11)
    say("qwen3-8b batch: qd_create_batch")
    m = qd.Model(mi, batch=B, paged=True, block_table=tbl, num_kv_blocks=nblk)
    for b in range(B):
        m.set_prompt_seq(b, stream)
    points = {}
    for tag in g["samples"]:
        kind, k = tag.split(":")
        points[int(k) if kind == "prefill" else P - 1 + int(k)] = tag
    last = P + G - 2
    preds = np.full((B, last + 1), -1, np.int32)
    lg = torch.empty((B, V), dtype=torch.float32, device="cuda")
    got = {}
    pos = 0
    for stop in sorted(set(points) | {last}):
        n = stop + 1 - pos
        seg = torch.full((B, n), -1, dtype=torch.int32, device="cuda")
        m.generate_batch([pos] * B, n, tokens=seg, logits_last=lg)
        preds[:, pos:stop + 1] = host(seg)
        if stop in points:
            got[points[stop]] = host(lg).copy()
        pos = stop + 1
        say(f"qwen3-8b batch: reached position {pos}")
    m.check()
    m.close()
    ref = np.asarray(g["tokens"], dtype=np.int32)
    worst = 0.0
    for b in range(B):
        gr = preds[b, P - 1:P - 1 + G]
        bad = np.nonzero(gr != ref)[0]
        record(f"qwen3-8b batch B={B} seq {b}: {G - len(bad)}/{G} teacher-forced greedy tokens equal"
               + (f" (first difference at step {int(bad[0])}, oracle margin {float(g['margins'][bad[0]]):.3e})"
                  if len(bad) else ""))
        assert len(bad) == 0
        for tag, lv in got.items():
            smp = g["samples"][tag]
            err = float(np.max(np.abs(lv[b][np.array(smp["idx"])] - np.array(smp["val"]))))
            err = max(err, float(np.max(np.abs(lv[b][np.array(smp["top_idx"])] - np.array(smp["top_val"])))))
            worst = max(worst, err)
    record(f"qwen3-8b batch B={B}: {len(got)} sampled positions x {B} sequences, worst logit error {worst:.3e}")
    assert worst <= LOGITS_BAR
