"""Pin of the oracle's whole decode step.

The oracle runs the tiny config one token at a time (sequential decode with a
KV cache).  The installed ``transformers`` Qwen3 implementation, loaded with
the same dequantised weights and run in f64, computes the same logits for the
whole prompt at once with a causal mask and no cache: a separate
implementation and a separate algorithm (full causal attention, not
incremental decode).  As shipped it computes RMSNorm statistics, the rotary
tables and (eager path) the softmax in f32 even for an f64 model, so it agrees
to f32 rounding; with the norm and rotary switched to the model's own dtype
(same formulas, no down-cast) and torch's SDPA for the attention, it agrees
to f64 rounding.
"""
import contextlib
import numpy as np
import pytest
import torch

import synth


def _hf_model(mi, oracle_lib, attn="eager"):
    from transformers import Qwen3Config, Qwen3ForCausalLM
    s = mi.shape
    cfg = Qwen3Config(vocab_size=s.vocab, hidden_size=s.hidden, intermediate_size=s.intermediate,
                      num_hidden_layers=s.layers, num_attention_heads=s.n_heads,
                      num_key_value_heads=s.n_kv, head_dim=s.head_dim, rope_theta=s.rope_theta,
                      rms_norm_eps=s.eps, tie_word_embeddings=s.tied,
                      max_position_embeddings=max(64, s.max_seq), attention_bias=False)
    cfg._attn_implementation = attn
    torch.manual_seed(0)
    m = Qwen3ForCausalLM(cfg).to(torch.float64).eval()
    T = lambda a: torch.tensor(np.asarray(a, dtype=np.float64))
    with torch.no_grad():
        m.model.embed_tokens.weight.copy_(T(oracle_lib.dequant(mi.embed)))
        for i, L in enumerate(mi.layers):
            ml = m.model.layers[i]
            ml.self_attn.q_proj.weight.copy_(T(oracle_lib.dequant(L.wq)))
            ml.self_attn.k_proj.weight.copy_(T(oracle_lib.dequant(L.wk)))
            ml.self_attn.v_proj.weight.copy_(T(oracle_lib.dequant(L.wv)))
            ml.self_attn.o_proj.weight.copy_(T(oracle_lib.dequant(L.wo)))
            ml.self_attn.q_norm.weight.copy_(T(L.q_norm))
            ml.self_attn.k_norm.weight.copy_(T(L.k_norm))
            ml.mlp.gate_proj.weight.copy_(T(oracle_lib.dequant(L.wgate)))
            ml.mlp.up_proj.weight.copy_(T(oracle_lib.dequant(L.wup)))
            ml.mlp.down_proj.weight.copy_(T(oracle_lib.dequant(L.wdown)))
            ml.input_layernorm.weight.copy_(T(L.attn_norm))
            ml.post_attention_layernorm.weight.copy_(T(L.ffn_norm))
        m.model.norm.weight.copy_(T(mi.final_norm))
        if not s.tied:
            m.lm_head.weight.copy_(T(oracle_lib.dequant(mi.lm_head)))
        # the same host-precomputed frequencies the oracle is given
        m.model.rotary_emb.inv_freq.copy_(torch.tensor(mi.inv_freq.astype(np.float64)))
    return m


@pytest.fixture(scope="module")
def tiny():
    return synth.make_model("tiny")


@contextlib.contextmanager
def _hf_in_f64():
    """Run transformers' Qwen3 RMSNorm and rotary tables in the input dtype."""
    from transformers.models.qwen3 import modeling_qwen3 as mq
    old_norm, old_rot = mq.Qwen3RMSNorm.forward, mq.Qwen3RotaryEmbedding.forward

    def norm(self, h):
        var = h.pow(2).mean(-1, keepdim=True)
        return self.weight * (h * torch.rsqrt(var + self.variance_epsilon))

    @torch.no_grad()
    def rot(self, x, position_ids):
        f = self.inv_freq.to(torch.float64)[None, :, None] * position_ids[:, None, :].to(torch.float64)
        emb = torch.cat((f, f), dim=1).transpose(1, 2)
        return emb.cos().to(x.dtype), emb.sin().to(x.dtype)

    mq.Qwen3RMSNorm.forward, mq.Qwen3RotaryEmbedding.forward = norm, rot
    try:
        yield
    finally:
        mq.Qwen3RMSNorm.forward, mq.Qwen3RotaryEmbedding.forward = old_norm, old_rot


def _hf_logits(mi, oracle_lib, attn="eager"):
    hf = _hf_model(mi, oracle_lib, attn)
    with torch.no_grad():
        return hf(torch.tensor(mi.prompt[None, :].astype(np.int64))).logits[0].numpy()


def test_sequential_decode_equals_full_causal_forward(oracle_lib, tiny):
    mi = tiny
    om = oracle_lib.Model(mi, kv_round=False)
    ours = np.stack([om.step(int(t), p) for p, t in enumerate(mi.prompt)])
    ref32 = _hf_logits(mi, oracle_lib)
    with _hf_in_f64():
        # torch's SDPA keeps the softmax in f64 (the eager path casts it to f32)
        ref64 = _hf_logits(mi, oracle_lib, attn="sdpa")
    scale = np.abs(ref64).max()
    assert np.max(np.abs(ours - ref64)) <= 1e-12 * scale
    assert np.max(np.abs(ours - ref32)) <= 1e-6 * scale
    # a wrong step would be far outside either bound
    assert np.abs(ref64[1:] - ref64[:-1]).max(axis=1).min() > 0.1 * scale


def test_f16_kv_cache_rounding(oracle_lib, tiny):
    """kv_round stores K/V as binary16 and changes logits only at the level of
    that rounding."""
    mi = tiny
    a = oracle_lib.Model(mi, kv_round=True)
    b = oracle_lib.Model(mi, kv_round=False)
    la = [a.step(int(t), p) for p, t in enumerate(mi.prompt[:6])]
    lb = [b.step(int(t), p) for p, t in enumerate(mi.prompt[:6])]
    for L in range(mi.shape.layers):
        for p in range(6):
            for g in range(mi.shape.n_kv):
                for which in (0, 1):
                    kr = a.kv(L, p, g, which)
                    assert np.array_equal(kr, kr.astype(np.float16).astype(np.float64))
                    if L == 0:
                        # layer 0's K/V depend only on the token: the rounded
                        # model stores exactly the binary16 of the unrounded one
                        kf = b.kv(L, p, g, which)
                        assert np.array_equal(kr, kf.astype(np.float16).astype(np.float64))
    d = max(np.abs(x - y).max() for x, y in zip(la, lb))
    assert 0 < d < 1e-2


def test_oracle_step_rejects_bad_inputs(oracle_lib, tiny):
    om = oracle_lib.Model(tiny)
    with pytest.raises(ValueError):
        om.step(tiny.shape.vocab, 0)
    with pytest.raises(ValueError):
        om.step(0, tiny.shape.max_seq)
    with pytest.raises(ValueError):
        om.step(-1, 0)


def test_generate_counts(oracle_lib, tiny):
    om = oracle_lib.Model(tiny)
    steps = []
    toks, margins, kept = oracle_lib.generate(om, tiny.prompt, 5, keep_logits_at=(0, 4),
                                              on_step=steps.append)
    P = tiny.shape.prompt_len
    assert len(toks) == 5 and len(margins) == 5 and set(kept) == {0, 4}
    assert steps == list(range(P + 5 - 1))
    assert toks[0] == int(np.argmax(kept[0].astype(np.float32)))


def test_fp8_cache_stores_e4m3_values(oracle_lib):
    """With kv_fp8 the oracle model stores e4m3(value / scale) * scale: every
    stored K value divided by k_scale (V by v_scale) is an e4m3 value, and it is
    the nearest one to the value the f64 step computed (the f64-kept cache)."""
    import synth
    mi = synth.make_model("tiny")
    ks, vs = 0.5, 0.125
    m8 = oracle_lib.Model(mi, kv_fp8=True, k_scale=ks, v_scale=vs)
    m64 = oracle_lib.Model(mi, kv_round=False)
    grid = oracle_lib.e4m3_to_f64(np.arange(256, dtype=np.uint8))
    grid = np.unique(grid[~np.isnan(grid)])
    for p, t in enumerate(mi.prompt[:6]):
        m8.step(int(t), p)
        m64.step(int(t), p)
    for layer in range(mi.shape.layers):
        for p in range(6):
            for g in range(mi.shape.n_kv):
                for which, sc in ((0, ks), (1, vs)):
                    got = m8.kv(layer, p, g, which) / sc
                    assert np.all(np.isin(got, grid))
                    # only layer 0 at position 0 is comparable: everything later reads
                    # the rounded cache through the attention
                    if p == 0 and layer == 0:
                        want = oracle_lib.e4m3_to_f64(oracle_lib.f64_to_e4m3(m64.kv(layer, p, g, which) / sc))
                        assert np.array_equal(got, want)



# ----------------------------------------------------------------- attention output gate
# inferencelayer cuda_llm.rs page, Cfg::attn_out_gate and the loader's q|k|v|gate
# rows: a second projection of the normed input, sigmoid, applied to the
# attention result before the o-projection.

def _one_layer_gated(oracle_lib):
    import dataclasses
    import synth
    shape = dataclasses.replace(synth.MODELS["tiny"], layers=1, name="tiny-1l")
    return synth.make_model(shape, attn_out_gate=True)


def test_attn_gate_first_step_closed_form(oracle_lib):
    """Position 0 of a one-layer gated model in plain numpy f64: the attention
    over one key is V[0] (rounded to f16 as stored), so the step is embedding,
    RMSNorm, the projections, the gate sigmoid(Wag h) on V, o-projection,
    residual, SwiGLU MLP, final norm and LM head."""
    mi = _one_layer_gated(oracle_lib)
    s, L = mi.shape, mi.layers[0]
    D = oracle_lib.dequant
    tok = int(mi.prompt[0])
    x = D(mi.embed)[tok]

    def rms(v, w):
        return v / np.sqrt(np.mean(v * v) + s.eps) * w.astype(np.float64)

    h = rms(x, L.attn_norm)
    v = D(L.wv) @ h
    v16 = oracle_lib.f16_to_f64(oracle_lib.f64_to_f16(v))
    gate = D(L.attn_gate) @ h
    hd, grp = s.head_dim, s.n_heads // s.n_kv
    att = np.concatenate([v16[(hh // grp) * hd:(hh // grp + 1) * hd] for hh in range(s.n_heads)])
    att = att / (1.0 + np.exp(-gate))
    x = x + D(L.wo) @ att
    h2 = rms(x, L.ffn_norm)
    g, u = D(L.wgate) @ h2, D(L.wup) @ h2
    x = x + D(L.wdown) @ (g / (1.0 + np.exp(-g)) * u)
    ref = D(mi.lm_head) @ rms(x, mi.final_norm)
    import dataclasses
    got = oracle_lib.Model(mi).step(tok, 0)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12)
    # and the gate matters: the ungated model differs
    ungated = oracle_lib.Model(dataclasses.replace(
        mi, layers=[dataclasses.replace(L, attn_gate=None)])).step(tok, 0)
    assert np.max(np.abs(ungated - got)) > 1e-3


def test_attn_gate_zero_is_half(oracle_lib):
    """A gate of zero weights gives sigmoid(0) = 1/2 everywhere, which equals the
    ungated model with every o-projection scale halved (exact in f64)."""
    import dataclasses
    import synth
    mi = synth.make_model("tiny", attn_out_gate=True)
    layers_g, layers_h = [], []
    for L in mi.layers:
        zero = synth.Q4Matrix(np.zeros_like(L.attn_gate.d), L.attn_gate.qs)
        layers_g.append(dataclasses.replace(L, attn_gate=zero))
        dh = (L.wo.d.view(np.float16) / np.float16(2)).view(np.uint16)   # exact: normal scales
        assert np.array_equal(dh.view(np.float16).astype(np.float64) * 2,
                              L.wo.d.view(np.float16).astype(np.float64))
        layers_h.append(dataclasses.replace(L, attn_gate=None, wo=synth.Q4Matrix(dh, L.wo.qs)))
    mg = oracle_lib.Model(dataclasses.replace(mi, layers=layers_g))
    mh = oracle_lib.Model(dataclasses.replace(mi, layers=layers_h))
    for p, t in enumerate(mi.prompt[:8]):
        assert np.array_equal(mg.step(int(t), p), mh.step(int(t), p))


# ----------------------------------------------------------------- untied head, partial rotary
# The whole step as a separate numpy f64 program: full-sequence causal
# forward with no cache, written from the definition (inferencelayer
# cuda_llm.rs page, CudaQwen3::step and Cfg: rot_dim, tied embeddings;
# memra-engine qwen4exp_gpu.rs page, its host rotary twin: pairs (i, i + rot/2)
# over the first rot dims with theta^(-2i/rot), the other dims unchanged).
# It shares nothing with qd_oracle.c: its own q4_0 decode, norms, rotary,
# attention and MLP.

def _np_dequant(W) -> np.ndarray:
    d = np.asarray(W.d, dtype=np.uint16).view(np.float16).astype(np.float64)
    qs = np.asarray(W.qs, dtype=np.uint8)
    codes = np.concatenate([qs & 15, qs >> 4], axis=2).astype(np.float64)   # elements 0..15, 16..31
    return ((codes - 8.0) * d[:, :, None]).reshape(d.shape[0], d.shape[1] * 32)


def _np_forward(mi) -> np.ndarray:
    """Logits of every prompt position, f64, no K/V rounding."""
    s = mi.shape
    H, hd, nq, nkv = s.hidden, s.head_dim, s.n_heads, s.n_kv
    rot, half = s.rot_dim, s.rot_dim // 2
    P = len(mi.prompt)

    def rms(v, w):
        return v / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + s.eps) * np.asarray(w, np.float64)

    pos = np.arange(P, dtype=np.float64)[:, None]
    ang = pos * np.asarray(mi.inv_freq[:half], dtype=np.float32).astype(np.float64)[None, :]
    cos, sin = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]   # [P, 1, half]

    def rotary(t):   # t [P, heads, hd]
        out = t.copy()
        a, b = t[..., :half], t[..., half:rot]
        out[..., :half] = a * cos - b * sin
        out[..., half:rot] = a * sin + b * cos
        return out

    x = _np_dequant(mi.embed)[np.asarray(mi.prompt)]
    mask = np.tril(np.ones((P, P), dtype=bool))
    for L in mi.layers:
        h = rms(x, L.attn_norm)
        q = (h @ _np_dequant(L.wq).T).reshape(P, nq, hd)
        k = (h @ _np_dequant(L.wk).T).reshape(P, nkv, hd)
        v = (h @ _np_dequant(L.wv).T).reshape(P, nkv, hd)
        if s.qk_norm:
            q, k = rms(q, L.q_norm), rms(k, L.k_norm)
        q, k = rotary(q), rotary(k)
        att = np.empty((P, nq, hd))
        for hh in range(nq):
            g = hh // (nq // nkv)
            sc = (q[:, hh] @ k[:, g].T) / np.sqrt(hd)
            sc = np.where(mask, sc, -np.inf)
            p = np.exp(sc - sc.max(axis=1, keepdims=True))
            att[:, hh] = (p / p.sum(axis=1, keepdims=True)) @ v[:, g]
        x = x + att.reshape(P, nq * hd) @ _np_dequant(L.wo).T
        h2 = rms(x, L.ffn_norm)
        gt, up = h2 @ _np_dequant(L.wgate).T, h2 @ _np_dequant(L.wup).T
        x = x + (gt / (1.0 + np.exp(-gt)) * up) @ _np_dequant(L.wdown).T
    head = mi.embed if s.tied else mi.lm_head
    return rms(x, mi.final_norm) @ _np_dequant(head).T


@pytest.mark.parametrize("name", ["tiny", "tiny-untied", "tiny-rot32"])
def test_sequential_decode_equals_numpy_causal_forward(oracle_lib, name):
    """The oracle's sequential decode (K/V kept in f64) against the numpy
    full-sequence forward, for the tiny decoder, its untied-head variant and
    its partial-rotary (rot_dim 32 of head_dim 64) variant."""
    mi = synth.make_model(name)
    om = oracle_lib.Model(mi, kv_round=False)
    ours = np.stack([om.step(int(t), p) for p, t in enumerate(mi.prompt)])
    ref = _np_forward(mi)
    scale = np.abs(ref).max()
    assert np.max(np.abs(ours - ref)) <= 1e-11 * scale


def test_untied_head_equals_transformers(oracle_lib):
    """The untied-head tiny decoder against the installed transformers Qwen3
    (tie_word_embeddings=False, its own lm_head weights), in f64."""
    mi = synth.make_model("tiny-untied")
    assert not mi.shape.tied and mi.lm_head is not mi.embed
    om = oracle_lib.Model(mi, kv_round=False)
    ours = np.stack([om.step(int(t), p) for p, t in enumerate(mi.prompt)])
    with _hf_in_f64():
        ref = _hf_logits(mi, oracle_lib, attn="sdpa")
    assert np.max(np.abs(ours - ref)) <= 1e-12 * np.abs(ref).max()
    # the head matters: the tied model's logits are far from these
    tied = synth.make_model("tiny")
    ot = oracle_lib.Model(tied, kv_round=False)
    lt = np.stack([ot.step(int(t), p) for p, t in enumerate(tied.prompt)])
    assert np.max(np.abs(lt - ours)) > 0.1 * np.abs(ref).max()


def test_partial_rotary_leaves_tail_dims(oracle_lib):
    """With rot_dim 32 of 64 the rotary changes the logits (the variant differs
    from the full-rotary model with the same weights), yet a model whose
    frequencies are all zero equals one with rot_dim 0 (nothing turns)."""
    import dataclasses
    mi = synth.make_model("tiny-rot32")
    full = synth.make_model("tiny")
    a = oracle_lib.Model(mi, kv_round=False)
    b = oracle_lib.Model(full, kv_round=False)
    la = np.stack([a.step(int(t), p) for p, t in enumerate(mi.prompt[:6])])
    lb = np.stack([b.step(int(t), p) for p, t in enumerate(full.prompt[:6])])
    assert np.array_equal(la[0], lb[0])            # position 0: no rotation anywhere
    assert np.max(np.abs(la[1:] - lb[1:])) > 1e-3  # later positions: the widths differ
    z = dataclasses.replace(mi, inv_freq=np.zeros_like(mi.inv_freq))
    z0 = dataclasses.replace(mi, shape=dataclasses.replace(mi.shape, rot_dim=0),
                             inv_freq=np.zeros(0, np.float32))
    oz, o0 = oracle_lib.Model(z, kv_round=False), oracle_lib.Model(z0, kv_round=False)
    for p, t in enumerate(mi.prompt[:6]):
        assert np.array_equal(oz.step(int(t), p), o0.step(int(t), p))
