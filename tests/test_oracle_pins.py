"""Pins of the f64 CPU oracle against things other than itself.

Each test fixes one piece of the oracle with a closed form, a hand-built
case, a library routine that computes the same quantity by another route
(numpy's binary16 conversion, a dense numpy matmul, torch's rms_norm and
scaled_dot_product_attention, complex multiplication for the rotary), or an
invariant.  The full-step test compares with the installed ``transformers``
Qwen3 implementation run in f64 over a whole causal sequence with no cache.
"""
import numpy as np
import pytest
import torch

import synth


# ----------------------------------------------------------------- binary16

def test_f16_decode_exhaustive_vs_numpy(oracle_lib):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle_lib.f16_to_f64(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zero kept
    assert np.signbit(ours[0x8000]) and not np.signbit(ours[0])


def test_f16_encode_vs_numpy(oracle_lib):
    rng = np.random.default_rng(0)
    vals = np.concatenate([
        rng.standard_normal(4000),
        rng.standard_normal(2000) * 1e-5,           # subnormal range
        rng.standard_normal(2000) * 3e4,            # near overflow
        rng.standard_normal(1000) * 1e-8,           # underflow to zero
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e9, -1e9,
                  2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25,
                  1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 2047.5, 2048.0 + 1.0, 2049.0]),
    ])
    # exact halfway points between neighbouring binary16 values (ties to even)
    h = np.arange(0x0400, 0x7bff, 97, dtype=np.uint16).view(np.float16).astype(np.float64)
    h2 = np.arange(0x0401, 0x7c00, 97, dtype=np.uint16).view(np.float16).astype(np.float64)
    vals = np.concatenate([vals, (h + h2) / 2, -(h + h2) / 2])
    ours = oracle_lib.f64_to_f16(vals)
    ref = vals.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


# ----------------------------------------------------------------- q4_0

def _block(d_bits, codes):
    """One q4_0 row of one block from 32 codes (test-local packer)."""
    codes = np.asarray(codes, dtype=np.uint8)
    qs = (codes[:16] | (codes[16:] << 4)).astype(np.uint8)
    return synth.Q4Matrix(np.array([[d_bits]], dtype=np.uint16), qs.reshape(1, 1, 16))


def test_dequant_hand_block(oracle_lib):
    # byte j = j (low nibble) | (15 - j) << 4 (high nibble), d = 1.0
    qs = np.array([j | ((15 - j) << 4) for j in range(16)], dtype=np.uint8).reshape(1, 1, 16)
    W = synth.Q4Matrix(np.array([[0x3C00]], dtype=np.uint16), qs)
    v = oracle_lib.dequant(W)[0]
    assert list(v[:16]) == [j - 8 for j in range(16)]
    assert list(v[16:]) == [7 - j for j in range(16)]
    # d = -2.0 and a subnormal d = 2^-24
    W2 = synth.Q4Matrix(np.array([[0xC000]], dtype=np.uint16), qs)
    assert list(oracle_lib.dequant(W2)[0][:4]) == [16.0, 14.0, 12.0, 10.0]
    W3 = synth.Q4Matrix(np.array([[0x0001]], dtype=np.uint16), qs)
    assert oracle_lib.dequant(W3)[0][0] == -8 * 2.0 ** -24


def _pack_dense(codes, dbits):
    """Test-local packer: integer codes [R, K] and scale bits [R, K/32] -> q4_0."""
    R, K = codes.shape
    c = codes.reshape(R, K // 32, 32).astype(np.uint8)
    qs = (c[..., :16] | (c[..., 16:] << 4)).astype(np.uint8)
    return synth.Q4Matrix(dbits.astype(np.uint16), qs)


@pytest.mark.parametrize("R,K", [(1, 32), (3, 64), (17, 256), (64, 4096)])
def test_gemv_vs_dense_matmul(oracle_lib, R, K):
    rng = np.random.default_rng(R * 1000 + K)
    codes = rng.integers(0, 16, size=(R, K))
    dbits = (rng.standard_normal((R, K // 32)) * 0.01).astype(np.float16).view(np.uint16)
    W = _pack_dense(codes, dbits)
    dense = (codes - 8).astype(np.float64) * np.repeat(dbits.view(np.float16).astype(np.float64), 32, axis=1)
    x = rng.standard_normal(K).astype(np.float32)
    y = oracle_lib.gemv(W, x)
    ref = dense @ x.astype(np.float64)
    assert np.max(np.abs(y - ref)) <= 1e-13 * max(1.0, np.max(np.abs(ref)))
    # unit vectors pick columns: checks the column index of every element
    for c in [0, 1, 15, 16, 17, 31, K - 1]:
        e = np.zeros(K, dtype=np.float32)
        e[c] = 1.0
        assert np.array_equal(oracle_lib.gemv(W, e), dense[:, c])


def test_gemv_thread_count_invariant(oracle_lib):
    W, x = synth.random_gemv(11, 257, 512)
    a = oracle_lib.gemv(W, x, nthreads=1)
    b = oracle_lib.gemv(W, x, nthreads=7)
    assert np.array_equal(a, b)


def test_quantizer_round_trip(oracle_lib):
    """Harness quantizer: |dequant(quant(w)) - w| <= |d|/2 (plus the f16 scale
    rounding) except where the code clamps at 15."""
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((8, 256)) * 0.02).astype(np.float32)
    d, qs = synth.quantize_q4_0(w)
    W = synth.Q4Matrix(d, qs)
    back = oracle_lib.dequant(W)
    dd = np.repeat(d.view(np.float16).astype(np.float64), 32, axis=1)
    codes = np.concatenate([qs & 15, qs >> 4], axis=2).reshape(8, 256)
    err = np.abs(back - w)
    ok = (err <= np.abs(dd) * 0.5 * (1 + 1e-3) + 1e-12) | (codes == 15)
    assert ok.all()
    # the block's largest-magnitude element is represented exactly by code 0
    blk = w.reshape(8, 8, 32)
    i = np.abs(blk).argmax(axis=2)
    m = np.take_along_axis(blk, i[..., None], axis=2)[..., 0]
    assert np.allclose(back.reshape(8, 8, 32)[np.arange(8)[:, None], np.arange(8)[None, :], i],
                       d.view(np.float16).astype(np.float64) * -8)
    assert np.all(np.abs(m - d.view(np.float16).astype(np.float64) * -8) <= np.abs(m) * 1e-3)


# ----------------------------------------------------------------- RMSNorm

def test_rmsnorm_closed_form(oracle_lib):
    n, c, eps = 64, 0.37, 1e-6
    w = np.linspace(0.5, 1.5, n).astype(np.float32)
    y = oracle_lib.rmsnorm(np.full(n, c), w, eps)
    assert np.allclose(y, c / np.sqrt(c * c + eps) * w.astype(np.float64), rtol=1e-15, atol=0)


def test_rmsnorm_vs_torch(oracle_lib):
    rng = np.random.default_rng(5)
    for n in (64, 128, 4096):
        x = rng.standard_normal(n) * 3
        w = (1 + 0.1 * rng.standard_normal(n)).astype(np.float32)
        ref = torch.nn.functional.rms_norm(torch.tensor(x), (n,), torch.tensor(w, dtype=torch.float64),
                                           eps=1e-6).numpy()
        assert np.allclose(oracle_lib.rmsnorm(x, w, 1e-6), ref, rtol=1e-14, atol=1e-15)


# ----------------------------------------------------------------- rotary

def test_rope_identity_at_zero_and_norms(oracle_lib):
    rng = np.random.default_rng(6)
    hd = 128
    inv = synth.rope_inv_freq(1e6, hd)
    v = rng.standard_normal(hd)
    assert np.array_equal(oracle_lib.rope(v, hd, inv, 0), v)
    for pos in (1, 7, 2047, 32767):
        r = oracle_lib.rope(v, hd, inv, pos)
        half = hd // 2
        pn = v[:half] ** 2 + v[half:] ** 2
        rn = r[:half] ** 2 + r[half:] ** 2
        assert np.allclose(pn, rn, rtol=1e-13, atol=1e-14)


def test_rope_is_complex_rotation(oracle_lib):
    rng = np.random.default_rng(7)
    hd, rot = 128, 96           # partial rotary: the last 32 dims pass through
    inv = synth.rope_inv_freq(1e4, rot)
    v = rng.standard_normal(hd)
    pos = 123
    r = oracle_lib.rope(v, rot, inv, pos)
    half = rot // 2
    z = (v[:half] + 1j * v[half:rot]) * np.exp(1j * pos * inv.astype(np.float64))
    assert np.allclose(r[:half], z.real, rtol=0, atol=1e-13)
    assert np.allclose(r[half:rot], z.imag, rtol=0, atol=1e-13)
    assert np.array_equal(r[rot:], v[rot:])


def test_rope_relative_position(oracle_lib):
    rng = np.random.default_rng(8)
    hd = 64
    inv = synth.rope_inv_freq(1e6, hd)
    q, k = rng.standard_normal(hd), rng.standard_normal(hd)
    a = oracle_lib.rope(q, hd, inv, 40) @ oracle_lib.rope(k, hd, inv, 13)
    b = oracle_lib.rope(q, hd, inv, 40 + 500) @ oracle_lib.rope(k, hd, inv, 13 + 500)
    assert abs(a - b) <= 1e-11 * (np.linalg.norm(q) * np.linalg.norm(k))


# ----------------------------------------------------------------- attention

def _f16(x):
    return np.asarray(x, dtype=np.float16).view(np.uint16)


def _sdpa_ref(q, kc, vc, lens, scale):
    """torch SDPA (f64) per sequence, GQA by repeating kv heads."""
    B, nq, hd = q.shape
    nkv = kc.shape[1]
    out = np.zeros((B, nq, hd))
    for b in range(B):
        n = int(lens[b])
        if n == 0:
            continue
        K = torch.tensor(kc[b, :, :n].view(np.float16).astype(np.float64))
        V = torch.tensor(vc[b, :, :n].view(np.float16).astype(np.float64))
        K = K.repeat_interleave(nq // nkv, dim=0).contiguous()
        V = V.repeat_interleave(nq // nkv, dim=0).contiguous()
        Q = torch.tensor(q[b].astype(np.float64))[:, None, :]
        o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=scale)
        out[b] = o[:, 0, :].numpy()
    return out


def test_attention_vs_torch_sdpa_paged_and_contiguous(oracle_lib):
    a = synth.random_attn(21, 3, [1, 37, 200], nq=8, nkv=2, hd=64)
    scale = 1 / np.sqrt(64)
    paged = oracle_lib.attn_inputs(a)
    kc, vc = synth.contiguous_from_paged(a)
    contig = oracle_lib.attn_decode(a.q, kc, vc, a.kv_lens, a.nkv, scale, contig_max_kv=kc.shape[2])
    assert np.array_equal(paged, contig)          # paging is a permutation of storage
    ref = _sdpa_ref(a.q, kc, vc, a.kv_lens, scale)
    assert np.allclose(paged, ref, rtol=1e-12, atol=1e-13)


def test_attention_special_cases(oracle_lib):
    hd, nq, nkv = 64, 4, 4
    rng = np.random.default_rng(9)
    q = rng.standard_normal((1, nq, hd)).astype(np.float32)
    # kv_len 1 -> the single V row
    k = _f16(rng.standard_normal((1, nkv, 1, hd)))
    v = _f16(rng.standard_normal((1, nkv, 1, hd)))
    o = oracle_lib.attn_decode(q, k, v, [1], nkv, 0.125, contig_max_kv=1)
    assert np.array_equal(o[0], v[0, :, 0].view(np.float16).astype(np.float64))
    # identical keys -> mean of V
    n = 9
    kk = np.broadcast_to(k, (1, nkv, n, hd)).copy()
    vv = _f16(rng.standard_normal((1, nkv, n, hd)))
    o = oracle_lib.attn_decode(q, kk, vv, [n], nkv, 0.125, contig_max_kv=n)
    assert np.allclose(o[0], vv[0].view(np.float16).astype(np.float64).mean(axis=1), rtol=1e-14, atol=1e-15)
    # huge logits stay finite and pick the winning key's V
    big = np.zeros((1, nkv, 3, hd), dtype=np.float16)
    big[0, :, 1, 0] = 60000.0
    vals = _f16(rng.standard_normal((1, nkv, 3, hd)))
    qb = np.zeros((1, nq, hd), dtype=np.float32)
    qb[0, :, 0] = 1.0
    o = oracle_lib.attn_decode(qb, big.view(np.uint16), vals, [3], nkv, 1.0, contig_max_kv=3)
    assert np.array_equal(o[0], vals[0, :, 1].view(np.float16).astype(np.float64))
    # kv_len 0 -> zeros (reading: an empty context attends to nothing)
    o = oracle_lib.attn_decode(q, k, v, [0], nkv, 0.125, contig_max_kv=1)
    assert np.all(o == 0)


def test_attention_softmax_rows_sum_to_one(oracle_lib):
    """With V[t] = e_t (one-hot, kv_len <= head_dim) the output of head h is its
    softmax row over the keys: non-negative, summing to 1 (within f64 rounding),
    equal to exp(s - max) / sum exp(s - max) of the scores, also for scores near
    +-1e3; with V = all ones every output element is that sum."""
    rng = np.random.default_rng(17)
    hd, nq, nkv, n = 64, 4, 2, 40
    for amp in (1.0, 1e3):
        q = (rng.standard_normal((1, nq, hd)) * amp).astype(np.float32)
        k = _f16(rng.standard_normal((1, nkv, n, hd)))
        eye = np.zeros((1, nkv, n, hd))
        eye[0, :, np.arange(n), np.arange(n)] = 1.0
        o = oracle_lib.attn_decode(q, k, _f16(eye), [n], nkv, 0.125, contig_max_kv=n)[0]
        p = o[:, :n]
        assert np.all(o[:, n:] == 0) and np.all(p >= 0)
        assert np.allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-14)
        kf = k.view(np.float16).astype(np.float64)[0]
        for h in range(nq):
            sc = 0.125 * kf[h // (nq // nkv)] @ q[0, h].astype(np.float64)
            e = np.exp(sc - sc.max())
            assert np.allclose(p[h], e / e.sum(), rtol=1e-12, atol=1e-300)
        ones = oracle_lib.attn_decode(q, k, _f16(np.ones((1, nkv, n, hd))), [n], nkv, 0.125,
                                      contig_max_kv=n)[0]
        assert np.allclose(ones, 1.0, rtol=0, atol=1e-14)


def test_attention_gqa_equals_repeated_mha(oracle_lib):
    a = synth.random_attn(22, 1, [70], nq=8, nkv=2, hd=64, shuffle=False)
    scale = 0.125
    kc, vc = synth.contiguous_from_paged(a)
    g = oracle_lib.attn_decode(a.q, kc, vc, a.kv_lens, 2, scale, contig_max_kv=kc.shape[2])
    k4 = np.repeat(kc, 4, axis=1)
    v4 = np.repeat(vc, 4, axis=1)
    m = oracle_lib.attn_decode(a.q, k4, v4, a.kv_lens, 8, scale, contig_max_kv=kc.shape[2])
    assert np.array_equal(g, m)


def test_split_kv_merge_equals_unsplit(oracle_lib):
    """The split-KV combine rule (inferencelayer cuda_llm.rs page, attn_reduce;
    ferrum-kernels cuda_decode.rs page, flash_decode_attention phase 2): the
    oracle's attention over each key range s, with its range max m_s and
    softmax denominator l_s, merged as
        out = sum_s e^(m_s - M) l_s out_s / sum_s e^(m_s - M) l_s,  M = max m_s,
    equals the oracle's attention over the whole range, for uneven splits."""
    rng = np.random.default_rng(31)
    hd, nq, nkv, n = 64, 4, 2, 203
    scale = 1 / np.sqrt(hd)
    q = rng.standard_normal((1, nq, hd)).astype(np.float32)
    k = _f16(rng.standard_normal((1, nkv, n, hd)) * 2.0)
    v = _f16(rng.standard_normal((1, nkv, n, hd)))
    full = oracle_lib.attn_decode(q, k, v, [n], nkv, scale, contig_max_kv=n)[0]
    kf = k.view(np.float16).astype(np.float64)[0]
    for cuts in ([0, 64, 128, 192, n], [0, 1, 2, 150, n], [0, 100, n]):
        num = np.zeros((nq, hd))
        den = np.zeros(nq)
        ms, ls, outs = [], [], []
        for a, b in zip(cuts[:-1], cuts[1:]):
            ks = np.ascontiguousarray(k[:, :, a:b])
            vs = np.ascontiguousarray(v[:, :, a:b])
            outs.append(oracle_lib.attn_decode(q, ks, vs, [b - a], nkv, scale, contig_max_kv=b - a)[0])
            sc = np.stack([scale * kf[h // (nq // nkv), a:b] @ q[0, h].astype(np.float64) for h in range(nq)])
            m = sc.max(axis=1)
            ms.append(m)
            ls.append(np.exp(sc - m[:, None]).sum(axis=1))
        M = np.max(ms, axis=0)
        for m, l, o in zip(ms, ls, outs):
            f = np.exp(m - M) * l
            num += f[:, None] * o
            den += f
        assert np.allclose(num / den[:, None], full, rtol=1e-13, atol=1e-14)


# ----------------------------------------------------------------- greedy

def test_greedy_lowest_index_on_ties(oracle_lib):
    lg = np.array([0.1, 2.0, -1.0, 2.0, 1.9999])
    t, margin = oracle_lib.greedy_pick(lg)
    assert t == 1 and margin == 0.0
    # the pick happens on f32-rounded logits: an f64-only difference is a tie
    lg = np.array([1.0, 1.0 + 1e-12])
    assert oracle_lib.greedy_pick(lg)[0] == 0


# --------------------------------------------------------------------------- rotary scaling
# inferencelayer cuda_llm.rs page, Cfg::rope_inv_freq: default / linear / llama3.

def test_rope_inv_freq_default_closed_form(oracle_lib):
    f = oracle_lib.rope_inv_freq(1e6, 128)
    assert f.shape == (64,)
    assert f[0] == 1.0
    # f_i = theta^(-2i/rot): consecutive ratios are all theta^(-2/rot)
    np.testing.assert_allclose(f[1:] / f[:-1], 1e6 ** (-2.0 / 128), rtol=1e-13)
    np.testing.assert_allclose(f[32], 1e6 ** -0.5, rtol=1e-13)


def test_rope_inv_freq_factor_one_is_identity(oracle_lib):
    base = oracle_lib.rope_inv_freq(5e5, 64)
    for sc in ("linear", "llama3"):
        np.testing.assert_allclose(oracle_lib.rope_inv_freq(5e5, 64, sc, factor=1.0), base, rtol=1e-15)


def test_rope_inv_freq_linear_divides(oracle_lib):
    base = oracle_lib.rope_inv_freq(1e4, 128)
    np.testing.assert_allclose(oracle_lib.rope_inv_freq(1e4, 128, "linear", factor=4.0), base / 4.0,
                               rtol=1e-15)


def test_rope_inv_freq_llama3_regions_and_continuity(oracle_lib):
    theta, rot, fac, lo, hi, orig = 5e5, 128, 8.0, 1.0, 4.0, 8192.0
    base = oracle_lib.rope_inv_freq(theta, rot)
    f = oracle_lib.rope_inv_freq(theta, rot, "llama3", fac, lo, hi, orig)
    wl = 2 * np.pi / base
    short, long_ = wl < orig / hi, wl > orig / lo
    mid = ~short & ~long_
    assert short.any() and long_.any() and mid.any()
    np.testing.assert_allclose(f[short], base[short], rtol=1e-15)        # high frequencies kept
    np.testing.assert_allclose(f[long_], base[long_] / fac, rtol=1e-15)  # low frequencies scaled
    # in between: strictly between f/factor and f
    assert np.all(f[mid] < base[mid]) and np.all(f[mid] > base[mid] / fac)
    # the blend is continuous at both edges: evaluate the rule at wavelengths
    # on either side of each boundary (theta chosen so that f_1 sits on it)
    for edge in (orig / lo, orig / hi):
        for eps in (1e-9, -1e-9):
            w = edge * (1 + eps)
            th = (2 * np.pi / w) ** (-rot / 2.0)   # f_1 = th^(-2/rot) = 2 pi / w
            g = oracle_lib.rope_inv_freq(th, rot, "llama3", fac, lo, hi, orig)[1]
            b = oracle_lib.rope_inv_freq(th, rot)[1]
            expect = b / fac if edge == orig / lo else b
            assert abs(g - expect) <= 1e-6 * b
    # the scaled frequencies still decrease with i
    assert np.all(np.diff(f) < 0)


def test_rope_inv_freq_unknown_type_refused(oracle_lib):
    with pytest.raises(ValueError):
        oracle_lib.rope_inv_freq(1e4, 64, "yarn", factor=2.0)


# --------------------------------------------------------------------------- fp8 e4m3 (KV cache)

def test_e4m3_decode_all_codes_vs_torch(oracle_lib):
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle_lib.e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan) and nan.sum() == 2
    assert np.array_equal(ours[~nan], ref[~nan])
    # closed forms: 1.0 = 0x38, max 448 = 0x7e, smallest subnormal 2^-9 = 0x01
    assert ours[0x38] == 1.0 and ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9
    assert ours[0xB8] == -1.0 and ours[0x80] == 0.0 and np.signbit(ours[0x80])


def test_e4m3_harness_quantizer_vs_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 0.1, 1.0, 30.0)])
    ours = synth.quantize_e4m3(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    # ties go to the even code: 1 + 1/16 lies halfway between 0x38 and 0x39
    assert synth.quantize_e4m3(np.array([1.0 + 1 / 16]))[0] == 0x38
    assert synth.quantize_e4m3(np.array([1.0 + 3 / 16]))[0] == 0x3A
    # saturation (torch would give NaN there)
    assert list(synth.quantize_e4m3(np.array([1e4, -1e4, 449.0]))) == [0x7E, 0xFE, 0x7E]


def test_attn_decode_e4m3_scales(oracle_lib):
    """The fp8 attention is the f16 attention of the decoded values with K
    scaled into the scores and V into the outputs: check against an explicit
    f64 softmax on a small case."""
    rng = np.random.default_rng(3)
    B, nq, nkv, hd, T = 1, 4, 2, 64, 37
    q = rng.standard_normal((B, nq, hd)).astype(np.float32)
    k8 = synth.quantize_e4m3(rng.standard_normal((B, nkv, T, hd)))
    v8 = synth.quantize_e4m3(rng.standard_normal((B, nkv, T, hd)))
    ks, vs, sc = 0.75, 1.5, 0.125
    got = oracle_lib.attn_decode_e4m3(q, k8, v8, np.array([T], np.int32), nkv, sc, ks, vs,
                                      contig_max_kv=T)
    K = oracle_lib.e4m3_to_f64(k8) * ks
    V = oracle_lib.e4m3_to_f64(v8) * vs
    for h in range(nq):
        g = h // (nq // nkv)
        s_ = K[0, g] @ q[0, h].astype(np.float64) * sc
        p_ = np.exp(s_ - s_.max())
        p_ /= p_.sum()
        np.testing.assert_allclose(got[0, h], p_ @ V[0, g], rtol=1e-12, atol=1e-14)


def test_e4m3_c_codec_vs_torch(oracle_lib):
    """The C oracle's e4m3 decode (all codes) and encode (round to nearest even,
    ties to even codes, in-range values) against torch float8_e4m3fn; saturation
    by closed form."""
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle_lib.e4m3_to_f64_c(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(3000) * s for s in (1e-3, 0.05, 1.0, 40.0)])
    # every exact midpoint between neighbouring finite codes (ties)
    vals = np.sort(ours[~nan & (codes < 0x7F)])
    mids = (vals[1:] + vals[:-1]) / 2
    x = np.concatenate([x, mids, -mids, vals, -vals])
    enc = oracle_lib.f64_to_e4m3(x)
    ref_enc = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(enc, ref_enc)
    assert list(oracle_lib.f64_to_e4m3(np.array([449.0, 1e6, -1e6]))) == [0x7E, 0x7E, 0xFE]
