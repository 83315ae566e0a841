"""GQA decode attention through the C ABI (qd_attn_decode) against the f64 oracle."""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import dev, host, normwise, say

pytestmark = pytest.mark.gpu

ATTN_TOL = 2e-5   # normwise, f32 softmax/accumulation vs f64


def _run(a: synth.AttnInputs, paged=True, workspace=None, contig=None, scale=None):
    import torch
    import token_decode_q4_amd as qd
    scale = 1.0 / np.sqrt(a.hd) if scale is None else scale
    out = torch.full((a.B, a.nq, a.hd), float("nan"), dtype=torch.float32, device="cuda")
    max_kv = max(1, a.max_kv_len)
    if workspace is None:
        nbytes = qd.attn_workspace_bytes(a.B, a.nq, a.nkv, a.hd, max_kv)
        workspace = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    if paged:
        qd.attn_decode(dev(a.q), dev(a.k_pool), dev(a.v_pool), dev(a.kv_lens), max_kv, a.nkv,
                       scale, out, workspace, block_tables=dev(a.block_tables))
    else:
        kc, vc = contig if contig is not None else synth.contiguous_from_paged(a, max_kv)
        qd.attn_decode(dev(a.q), dev(kc), dev(vc), dev(a.kv_lens), max_kv, a.nkv, scale, out,
                       workspace)
    return host(out), workspace


@pytest.mark.parametrize("name", sorted(synth.ATTN_CASES))
def test_attention_config_cases_full(name):
    say(f"attention case {name}")
    a = synth.attn_case(name)
    ref = oracle.attn_inputs(a)
    got, _ = _run(a)
    err = normwise(got, ref)
    say(f"attention {name}: kv_lens {a.kv_lens.tolist()[:8]} normwise err {err:.3e}")
    assert np.all(np.isfinite(got))
    assert err <= ATTN_TOL


@pytest.mark.parametrize("hd,nq,nkv", [(128, 32, 8), (128, 16, 8), (128, 8, 8), (64, 4, 2),
                                       (128, 16, 2), (64, 8, 1)])
def test_attention_ragged_lengths(hd, nq, nkv):
    lens = [0, 1, 15, 16, 17, 63, 64, 65, 200, 1000]
    say(f"attention ragged hd={hd} nq={nq} nkv={nkv} lens={lens}")
    a = synth.random_attn(31 + hd + nq, len(lens), lens, nq=nq, nkv=nkv, hd=hd)
    ref = oracle.attn_inputs(a)
    got, _ = _run(a)
    assert np.all(got[0] == 0)            # kv_len 0 -> zeros
    assert normwise(got, ref) <= ATTN_TOL


def test_attention_two_long_sequences():
    """Two sequences of 20 001 and 32 768 keys (32 q / 8 kv heads of 128): with
    several sequences the grid holds 2048 workgroups, 128 key splits per head,
    so the merge takes 16 splits per thread group in each of two load rounds."""
    lens = [20001, 32768]
    a = synth.random_attn(97, len(lens), lens, nq=32, nkv=8, hd=128)
    ref = oracle.attn_inputs(a)
    got, _ = _run(a)
    err = normwise(got, ref)
    say(f"attention two long sequences: normwise err {err:.3e}")
    assert err <= ATTN_TOL


def test_attention_paged_equals_contiguous_bitwise():
    a = synth.random_attn(41, 3, [5, 130, 777], nq=32, nkv=8, hd=128)
    p, _ = _run(a, paged=True)
    c, _ = _run(a, paged=False)
    assert np.array_equal(p, c)


def test_attention_ignores_unused_slots():
    """Slots past kv_len in a sequence's last block hold NaN; they must not leak."""
    a = synth.random_attn(42, 2, [17, 40], nq=8, nkv=2, hd=128)
    ref = oracle.attn_inputs(a)
    k = a.k_pool.copy()
    v = a.v_pool.copy()
    for b, n in enumerate(a.kv_lens):
        lb = (int(n) - 1) // 16
        phys = a.block_tables[b, lb]
        used = int(n) - lb * 16
        k[phys, :, used:] = 0x7E00   # f16 NaN
        v[phys, :, used:] = 0x7E00
    a2 = synth.AttnInputs(a.q, k, v, a.block_tables, a.kv_lens, a.nq, a.nkv, a.hd, a.block)
    got, _ = _run(a2)
    assert np.all(np.isfinite(got))
    assert normwise(got, ref) <= ATTN_TOL


def test_attention_workspace_reuse():
    """The completion counters reset themselves: a second call on the same
    workspace (and a call with different lengths) is still exact."""
    a = synth.random_attn(43, 2, [300, 1000], nq=32, nkv=8, hd=128)
    r1, ws = _run(a)
    r2, _ = _run(a, workspace=ws)
    assert np.array_equal(r1, r2)
    b = synth.random_attn(44, 2, [999, 3], nq=32, nkv=8, hd=128)
    got, _ = _run(b, workspace=ws)
    assert normwise(got, oracle.attn_inputs(b)) <= ATTN_TOL


def test_attention_large_scores():
    """Large logits (scale 8): the max-subtracted softmax stays finite."""
    a = synth.random_attn(45, 1, [500], nq=32, nkv=8, hd=128)
    ref = oracle.attn_decode(a.q, a.k_pool, a.v_pool, a.kv_lens, a.nkv, 8.0,
                             block_tables=a.block_tables, block_size=16)
    got, _ = _run(a, scale=8.0)
    assert np.all(np.isfinite(got))
    assert normwise(got, ref) <= 1e-4


# --------------------------------------------------------------------------- fp8 e4m3 cache

KV8_SCALES = (0.625, 1.75)   # k_scale, v_scale (not powers of two)


def _run_kv8(a: synth.AttnInputs, k8, v8, paged=True, contig=None):
    import torch
    import token_decode_q4_amd as qd
    scale = 1.0 / np.sqrt(a.hd)
    out = torch.full((a.B, a.nq, a.hd), float("nan"), dtype=torch.float32, device="cuda")
    max_kv = max(1, a.max_kv_len)
    ws = torch.zeros(qd.attn_workspace_bytes(a.B, a.nq, a.nkv, a.hd, max_kv), dtype=torch.uint8,
                     device="cuda")
    ks, vs = KV8_SCALES
    if paged:
        qd.attn_decode_kv8(dev(a.q), dev(k8), dev(v8), dev(a.kv_lens), max_kv, a.nkv, scale, ks, vs,
                           out, ws, block_tables=dev(a.block_tables))
    else:
        kc, vc = contig
        qd.attn_decode_kv8(dev(a.q), dev(kc), dev(vc), dev(a.kv_lens), max_kv, a.nkv, scale, ks, vs,
                           out, ws)
    return host(out)


def _kv8_pools(a: synth.AttnInputs):
    """the case's K/V values (f16 N(0,1)) in e4m3 through the harness quantizer"""
    k = a.k_pool.view(np.float16).astype(np.float64)
    v = a.v_pool.view(np.float16).astype(np.float64)
    return synth.quantize_e4m3(k), synth.quantize_e4m3(v)


def _ref_kv8(a, k8, v8, paged=True, contig_max_kv=0):
    ks, vs = KV8_SCALES
    return oracle.attn_decode_e4m3(a.q, k8, v8, a.kv_lens, a.nkv, 1.0 / np.sqrt(a.hd), ks, vs,
                                   a.block_tables if paged else None, contig_max_kv=contig_max_kv)


@pytest.mark.parametrize("name", sorted(synth.ATTN_CASES))
def test_attention_kv8_config_cases_full(name):
    say(f"attention fp8 case {name}")
    a = synth.attn_case(name)
    k8, v8 = _kv8_pools(a)
    got = _run_kv8(a, k8, v8)
    err = normwise(got, _ref_kv8(a, k8, v8))
    say(f"attention fp8 {name}: normwise err {err:.3e}")
    assert np.all(np.isfinite(got))
    assert err <= ATTN_TOL


@pytest.mark.parametrize("hd,nq,nkv", [(128, 32, 8), (64, 4, 2), (128, 16, 2), (64, 8, 1),
                                       (128, 8, 8)])
def test_attention_kv8_ragged_and_contiguous(hd, nq, nkv):
    a = synth.random_attn(500 + hd + nq, 3, [0, 1, 37], nq=nq, nkv=nkv, hd=hd)
    k8, v8 = _kv8_pools(a)
    got = _run_kv8(a, k8, v8)
    ref = _ref_kv8(a, k8, v8)
    assert np.array_equal(got[0], np.zeros_like(got[0]))     # kv_len 0 -> zeros
    assert normwise(got, ref) <= ATTN_TOL
    # the same cache laid out contiguously: bitwise the same result
    kc, vc = synth.contiguous_from_paged(a, max(1, a.max_kv_len))
    kc8 = synth.quantize_e4m3(kc.view(np.float16).astype(np.float64))
    vc8 = synth.quantize_e4m3(vc.view(np.float16).astype(np.float64))
    got_c = _run_kv8(a, k8, v8, paged=False, contig=(kc8, vc8))
    assert np.array_equal(got, got_c)


def test_attention_kv8_graph_replays_equal_eager():
    """qd_attn_decode_kv8 captured in a graph, replayed several times with eager
    work and synchronisations between the replays: every replay equals the
    eager call (bitwise)."""
    import torch
    import token_decode_q4_amd as qd
    a = synth.random_attn(77, 2, [300, 1000], nq=32, nkv=8, hd=128)
    k8, v8 = _kv8_pools(a)
    ref = _run_kv8(a, k8, v8)
    max_kv = max(1, a.max_kv_len)
    ws = torch.zeros(qd.attn_workspace_bytes(a.B, a.nq, a.nkv, a.hd, max_kv), dtype=torch.uint8,
                     device="cuda")
    out = torch.full((a.B, a.nq, a.hd), float("nan"), dtype=torch.float32, device="cuda")
    q, K, V, L, T = dev(a.q), dev(k8), dev(v8), dev(a.kv_lens), dev(a.block_tables)
    ks, vs = KV8_SCALES
    s = torch.cuda.Stream()

    def call():
        qd.attn_decode_kv8(q, K, V, L, max_kv, a.nkv, 1.0 / np.sqrt(a.hd), ks, vs, out, ws,
                           block_tables=T, stream=s)

    with torch.cuda.stream(s):
        call()
        s.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            call()
    for _ in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), ref)
        _run_kv8(a, k8, v8)   # eager work between the replays
