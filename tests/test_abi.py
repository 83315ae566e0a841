"""The C ABI library without a GPU: it loads, exports every function the
header declares, and rejects bad arguments with an error code before any HIP
call (so these run on a machine with no GPU)."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def qd():
    import token_decode_q4_amd as qd
    qd.lib()
    return qd


def test_header_functions_exported(qd):
    hdr = open(os.path.join(ROOT, "include", "qd.h")).read()
    hdr = re.sub(r"/\*.*?\*/", "", hdr, flags=re.S)
    names = set(re.findall(r"\b(qd_[a-z0-9_]+)\s*\(", hdr))
    assert names == set(qd.EXPORTS)
    L = qd.lib()
    for n in names:
        assert hasattr(L, n), n
    # and the shared object's dynamic symbol table agrees
    import subprocess
    syms = subprocess.run(["nm", "-D", "--defined-only", qd.LIB_PATH], capture_output=True,
                          text=True, check=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}$", syms, re.M), n


def test_prefill_chunk(qd):
    # four groups of 16 positions: the matrix-core product's vectors
    assert qd.prefill_chunk() == 64


def test_gemv_validation(qd):
    L = qd.lib()
    p = C.c_void_p(16)
    assert L.qd_gemv_q4_0(None, p, p, p, 4, 32, None) == qd._native.QD_EINVAL
    assert L.qd_gemv_q4_0(p, p, p, p, 4, 33, None) == qd._native.QD_EINVAL
    assert L.qd_gemv_q4_0(p, p, p, p, -1, 32, None) == qd._native.QD_EINVAL
    assert L.qd_gemv_q4_0(p, p, p, p, 4, 32 * 100000, None) == qd._native.QD_EUNSUPPORTED
    assert L.qd_gemv_q4_0(p, C.c_void_p(17), p, p, 4, 32, None) == qd._native.QD_EINVAL
    assert b"aligned" in L.qd_last_error()


def test_gemv_batch_validation(qd):
    L = qd.lib()
    p = C.c_void_p(16)
    E, U = qd._native.QD_EINVAL, qd._native.QD_EUNSUPPORTED
    assert L.qd_gemv_q4_0_batch(None, p, p, p, 4, 32, 2, None) == E
    assert L.qd_gemv_q4_0_batch(p, p, p, p, 4, 33, 2, None) == E
    assert L.qd_gemv_q4_0_batch(p, p, p, p, -1, 32, 2, None) == E
    assert L.qd_gemv_q4_0_batch(p, p, p, p, 4, 32, 0, None) == E
    assert L.qd_gemv_q4_0_batch(p, p, p, p, 4, 32, 17, None) == E
    assert b"batch" in L.qd_last_error()
    assert L.qd_gemv_q4_0_batch(p, p, p, p, 4, 4096, -3, None) == E
    assert L.qd_gemv_q4_0_batch(p, p, C.c_void_p(20), p, 4, 32, 2, None) == E
    assert b"aligned" in L.qd_last_error()
    assert L.qd_gemv_q4_0_batch(p, p, p, p, 1 << 24, 64, 2, None) == U


def test_attention_validation(qd):
    L = qd.lib()
    p = 16
    A = qd._native.AttnArgs
    good = dict(q=p, k=p, v=p, block_tables=p, max_blocks_per_seq=4, block_size=16, kv_lens=p,
                max_kv_len=64, B=1, nq=32, nkv=8, head_dim=128, scale=0.1, out=p)
    ws = qd.attn_workspace_bytes(1, 32, 8, 128, 64)
    assert ws > 0

    def call(**kw):
        d = dict(good, **kw)
        return L.qd_attn_decode(C.byref(A(**d)), C.c_void_p(16), ws, None)

    assert call(nq=30) == qd._native.QD_EINVAL
    assert call(nq=48, nkv=4) == qd._native.QD_EUNSUPPORTED   # group of 12
    assert call(head_dim=96) == qd._native.QD_EUNSUPPORTED
    assert call(block_size=32) == qd._native.QD_EUNSUPPORTED
    assert call(max_blocks_per_seq=3) == qd._native.QD_EINVAL
    assert call(q=None) == qd._native.QD_EINVAL
    assert L.qd_attn_decode(C.byref(A(**good)), C.c_void_p(16), ws - 1, None) == qd._native.QD_EINVAL
    assert L.qd_attn_decode(None, C.c_void_p(16), ws, None) == qd._native.QD_EINVAL
    assert qd.attn_workspace_bytes(0, 32, 8, 128, 64) == 0


def _cfg_weights(qd, mi, **over):
    """Config/weights structs for `mi` with fields overridden (all host memory)."""
    N = qd._native
    s = mi.shape
    keep = []
    layers = (N.LayerWeights * s.layers)()
    for i, Lw in enumerate(mi.layers):
        ns = [np.ascontiguousarray(a, dtype=np.float32) for a in
              (Lw.attn_norm, Lw.ffn_norm, Lw.q_norm, Lw.k_norm)]
        keep.append(ns)
        layers[i] = N.LayerWeights(*[a.ctypes.data for a in ns],
                                   *[N._q4(m) for m in (Lw.wq, Lw.wk, Lw.wv, Lw.wo, Lw.wgate,
                                                         Lw.wup, Lw.wdown)])
    fn = np.ascontiguousarray(mi.final_norm, dtype=np.float32)
    inv = np.ascontiguousarray(mi.inv_freq, dtype=np.float32)
    keep += [fn, inv, layers]
    w = N.Weights(N._q4(mi.embed), N._q4(mi.lm_head), fn.ctypes.data, layers)
    f = dict(hidden=s.hidden, layers=s.layers, n_heads=s.n_heads, n_kv=s.n_kv,
             head_dim=s.head_dim, intermediate=s.intermediate, vocab=s.vocab, eps=s.eps,
             rot_dim=s.rot_dim, inv_freq=inv.ctypes.data, tied=int(s.tied),
             qk_norm=int(s.qk_norm), max_seq=s.max_seq, kv_paged=0, kv_block_size=16,
             num_kv_blocks=0, block_table=None, use_graph=1)
    f.update(over)
    return N.Config(**f), w, keep


@pytest.mark.parametrize("over,code", [
    (dict(n_kv=3), -1), (dict(head_dim=96), -4), (dict(rot_dim=63), -1), (dict(rot_dim=66), -1),
    (dict(hidden=0), -1), (dict(n_heads=12, n_kv=1), -4), (dict(kv_paged=1, kv_block_size=32), -4),
    (dict(kv_paged=1, num_kv_blocks=2), -1), (dict(inv_freq=None), -1), (dict(vocab=1000), -1),
    (dict(intermediate=512), -1), (dict(eps=-1.0), -1),
    (dict(kv_fp8=2), -1), (dict(kv_fp8=1, k_scale=0.0, v_scale=1.0), -1),
    (dict(kv_fp8=1, k_scale=1.0, v_scale=float("nan")), -1),
    (dict(kv_fp8=1, k_scale=1.0, v_scale=1.0, layer_kernel=1), -4),
    (dict(attn_out_gate=2), -1), (dict(attn_out_gate=1), -1),   # the tiny weights carry no gate
])
def test_create_validation(qd, over, code):
    mi = synth.make_model("tiny")
    cfg, w, keep = _cfg_weights(qd, mi, **over)
    h = C.c_void_p()
    rc = qd.lib().qd_create(C.byref(cfg), C.byref(w), None, C.byref(h))
    assert rc == code, qd.lib().qd_last_error()
    assert not h.value


def test_create_rejects_bad_block_table(qd):
    mi = synth.make_model("tiny")
    for tbl in ([0, 0, 1], [0, 1, 9], [-1, 1, 2]):
        t = np.array(tbl, dtype=np.int32)
        cfg, w, keep = _cfg_weights(qd, mi, kv_paged=1, num_kv_blocks=4, block_table=t.ctypes.data)
        h = C.c_void_p()
        assert qd.lib().qd_create(C.byref(cfg), C.byref(w), None, C.byref(h)) == qd._native.QD_EINVAL


def test_create_rejects_null_weight(qd):
    mi = synth.make_model("tiny")
    cfg, w, keep = _cfg_weights(qd, mi)
    w.layers[1].wdown.qs = None
    h = C.c_void_p()
    assert qd.lib().qd_create(C.byref(cfg), C.byref(w), None, C.byref(h)) == qd._native.QD_EINVAL
    assert b"layer 1 wdown" in qd.lib().qd_last_error()


def test_stream_read_validation(qd):
    L = qd.lib()
    p = C.c_void_p(16)
    assert L.qd_stream_read(None, 64, p, None) == qd._native.QD_EINVAL
    assert L.qd_stream_read(p, 0, p, None) == qd._native.QD_EINVAL
    assert L.qd_stream_read(p, 40, p, None) == qd._native.QD_EINVAL
    assert L.qd_stream_read(C.c_void_p(24), 64, p, None) == qd._native.QD_EINVAL
    assert b"aligned" in L.qd_last_error()
    assert qd.stream_read_groups(0) == 0 and qd.stream_read_groups(40) == 0
    assert qd.stream_read_groups(16) == 1
    assert qd.stream_read_groups(16 * 1024) == 1 and qd.stream_read_groups(16 * 1025) == 2
    assert qd.stream_read_groups(1 << 30) == 2048


def test_create_rejects_layer_kernel_for_unfit_model(qd):
    """layer_kernel = 1 needs head_dim 128, 4 query heads per kv head and K
    multiples of 2048: the tiny model (head_dim 64) is refused before any HIP
    call."""
    mi = synth.make_model("tiny")
    cfg, w, keep = _cfg_weights(qd, mi, layer_kernel=1)
    h = C.c_void_p()
    assert qd.lib().qd_create(C.byref(cfg), C.byref(w), None, C.byref(h)) == qd._native.QD_EUNSUPPORTED
    assert b"layer_kernel" in qd.lib().qd_last_error()


@pytest.mark.parametrize("case", [
    dict(theta=1e6, rot_dim=128),
    dict(theta=1e4, rot_dim=64, scaling="linear", factor=4.0),
    dict(theta=5e5, rot_dim=128, scaling="llama3", factor=8.0, low_freq_factor=1.0,
         high_freq_factor=4.0, original_max_pos=8192.0),
    dict(theta=1e6, rot_dim=64, scaling="llama3", factor=16.0, low_freq_factor=2.0,
         high_freq_factor=8.0, original_max_pos=64.0),
    dict(theta=1e6, rot_dim=32),
])
def test_rope_inv_freq_matches_oracle(qd, case):
    """qd_rope_inv_freq (host code in the library, no device work) against the
    f64 oracle of the same rule: equal to f32 rounding."""
    import oracle
    got = qd.rope_inv_freq(**case)
    ref = oracle.rope_inv_freq(**case)
    assert got.dtype == np.float32 and got.shape == ref.shape
    np.testing.assert_allclose(got.astype(np.float64), ref, rtol=2 ** -23, atol=0)


def test_rope_inv_freq_validation(qd):
    L = qd.lib()
    out = np.empty(64, dtype=np.float32)
    p = out.ctypes.data
    E, U = qd._native.QD_EINVAL, qd._native.QD_EUNSUPPORTED
    assert L.qd_rope_inv_freq(1e4, 64, 0, 1.0, 1.0, 4.0, 8192.0, None) == E
    assert L.qd_rope_inv_freq(1e4, 63, 0, 1.0, 1.0, 4.0, 8192.0, p) == E
    assert L.qd_rope_inv_freq(1e4, 0, 0, 1.0, 1.0, 4.0, 8192.0, p) == E
    assert L.qd_rope_inv_freq(1.0, 64, 0, 1.0, 1.0, 4.0, 8192.0, p) == E
    assert L.qd_rope_inv_freq(1e4, 64, 1, 0.0, 1.0, 4.0, 8192.0, p) == E
    assert L.qd_rope_inv_freq(1e4, 64, 2, 8.0, 4.0, 1.0, 8192.0, p) == E
    assert L.qd_rope_inv_freq(1e4, 64, 2, 8.0, 1.0, 4.0, 0.0, p) == E
    assert L.qd_rope_inv_freq(1e4, 64, 3, 2.0, 1.0, 4.0, 8192.0, p) == U
    assert b"not implemented" in L.qd_last_error()
    with pytest.raises(qd.QdError):
        qd.rope_inv_freq(1e4, 64, "yarn", 2.0)


def test_attention_noalloc_validation(qd):
    """The no-allocation attention refuses bad arguments and sizes beyond its
    scratch before any HIP call."""
    L = qd.lib()
    E, U = qd._native.QD_EINVAL, qd._native.QD_EUNSUPPORTED
    assert qd.attn_noalloc_max_bytes() == 8 << 20
    assert L.qd_attn_decode_noalloc(None, None) == E
    p = C.c_void_p(16)
    assert qd.attn_workspace_bytes(512, 64, 8, 128, 64) > qd.attn_noalloc_max_bytes()
    a = qd._native.AttnArgs(p, p, p, p, 4, 16, p, 64, 512, 64, 8, 128, 0.1, p)
    assert L.qd_attn_decode_noalloc(C.byref(a), None) == U
    assert b"scratch" in L.qd_last_error()
    a = qd._native.AttnArgs(p, p, p, p, 4, 16, p, 64, 1, 32, 8, 96, 0.1, p)   # head_dim 96
    assert L.qd_attn_decode_noalloc(C.byref(a), None) == U
    a = qd._native.AttnArgs(p, p, None, p, 4, 16, p, 64, 1, 32, 8, 128, 0.1, p)
    assert L.qd_attn_decode_noalloc(C.byref(a), None) == E


def test_attention_kv8_validation(qd):
    L = qd.lib()
    A = qd._native.AttnArgs
    E = qd._native.QD_EINVAL
    good = dict(q=16, k=16, v=16, block_tables=16, max_blocks_per_seq=4, block_size=16, kv_lens=16,
                max_kv_len=64, B=1, nq=32, nkv=8, head_dim=128, scale=0.1, out=16)

    def call(ks=1.0, vs=1.0, **kw):
        d = dict(good, **kw)
        a = A(*[d[n] for n, _ in A._fields_])
        return L.qd_attn_decode_kv8(C.byref(a), ks, vs, C.c_void_p(16), 1 << 30, None)

    assert call(ks=0.0) == E
    assert call(vs=-1.0) == E
    assert call(ks=float("inf")) == E
    assert b"scale" in L.qd_last_error()
    assert call(k=24) == E
    assert b"aligned" in L.qd_last_error()
    assert call(head_dim=96) == qd._native.QD_EUNSUPPORTED
    assert call(nq=12) == E                              # nq % nkv != 0
    assert call(nq=48) == qd._native.QD_EUNSUPPORTED     # GQA group 6



def test_gemv_experts_validation(qd):
    L = qd.lib()
    p = C.c_void_p(16)
    E, U = qd._native.QD_EINVAL, qd._native.QD_EUNSUPPORTED
    assert L.qd_gemv_q4_0_experts(p, p, None, 8, 2, p, p, 64, 64, None) == E
    assert L.qd_gemv_q4_0_experts(p, p, p, 0, 2, p, p, 64, 64, None) == E
    assert L.qd_gemv_q4_0_experts(p, p, p, 8, -1, p, p, 64, 64, None) == E
    assert L.qd_gemv_q4_0_experts(p, p, p, 8, 2, p, p, 64, 65, None) == E
    assert L.qd_gemv_q4_0_experts(p, p, p, 8, 70000, p, p, 64, 64, None) == U
    assert L.qd_gemv_q4_0_experts(p, p, p, 8, 2, p, p, 64, 32 * 100000, None) == U
    assert L.qd_gemv_q4_0_experts(p, C.c_void_p(18), p, 8, 2, p, p, 64, 64, None) == E
    assert b"aligned" in L.qd_last_error()


def test_model_entry_points_reject_null_model(qd):
    L = qd.lib()
    assert L.qd_set_prompt_seq(None, 0, None, 0, None) == qd._native.QD_EINVAL
    assert L.qd_generate_batch(None, None, 1, None, None, None) == qd._native.QD_EINVAL
    assert L.qd_decode_step_batch(None, None, None, None, None, None) == qd._native.QD_EINVAL
    assert L.qd_create_batch(None, None, 1, None, None) == qd._native.QD_EINVAL
    assert L.qd_create_batch(None, None, 4, None, None) == qd._native.QD_EINVAL
    assert L.qd_prefill(None, 0, 1, None, None) == qd._native.QD_EINVAL
    assert L.qd_generate(None, 0, 1, None, None, None) == qd._native.QD_EINVAL
