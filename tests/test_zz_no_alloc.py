"""The no-allocation attention entry point (qd_attn_decode_noalloc, for
callers that cannot allocate) against the workspace entry point
(qd_attn_decode): two calls in a row, the second smaller, each bitwise equal
to qd_attn_decode on the same inputs (the same kernels and split geometry;
only the partials' buffer differs) and within the attention bar of the f64
oracle."""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import dev, host, normwise, say

pytestmark = pytest.mark.gpu

ATTN_TOL = 2e-5


def _both(a: synth.AttnInputs):
    import torch
    import token_decode_q4_amd as qd
    scale = 1.0 / np.sqrt(a.hd)
    max_kv = max(1, a.max_kv_len)
    args = (dev(a.q), dev(a.k_pool), dev(a.v_pool), dev(a.kv_lens), max_kv, a.nkv, scale)
    tbl = dev(a.block_tables)
    ws = torch.zeros(qd.attn_workspace_bytes(a.B, a.nq, a.nkv, a.hd, max_kv), dtype=torch.uint8, device="cuda")
    ref = torch.full((a.B, a.nq, a.hd), float("nan"), dtype=torch.float32, device="cuda")
    got = torch.full_like(ref, float("nan"))
    qd.attn_decode(*args, ref, ws, block_tables=tbl)
    qd.attn_decode_noalloc(*args, got, block_tables=tbl)
    return host(ref), host(got)


def test_attn_noalloc_equals_workspace_entry_point():
    cases = [synth.attn_case("b1_kv4096"),                                  # 32 / 8 heads of 128
             synth.random_attn(41, 3, [700, 1, 96], nq=8, nkv=2, hd=64)]    # smaller, ragged
    for i, a in enumerate(cases):
        say(f"no-alloc attention call {i}: B {a.B} nq {a.nq} nkv {a.nkv} hd {a.hd} kv_lens {a.kv_lens.tolist()}")
        ref, got = _both(a)
        assert np.array_equal(ref, got), i
        err = normwise(got, oracle.attn_inputs(a))
        say(f"no-alloc attention call {i}: bitwise equal, normwise err vs oracle {err:.3e}")
        assert err <= ATTN_TOL


def test_attn_noalloc_refuses_sizes_above_its_scratch():
    import torch
    import token_decode_q4_amd as qd
    # 512 sequences of 64 heads: more split partials than the scratch holds
    B, nq, nkv, hd, kv = 512, 64, 8, 128, 64
    assert qd.attn_workspace_bytes(B, nq, nkv, hd, kv) > qd.attn_noalloc_max_bytes()
    q = torch.zeros((B, nq, hd), dtype=torch.float32, device="cuda")
    k = torch.zeros((1, nkv, 16, hd), dtype=torch.float16, device="cuda")
    lens = torch.ones(B, dtype=torch.int32, device="cuda")
    out = torch.full((B, nq, hd), float("nan"), dtype=torch.float32, device="cuda")
    tbl = torch.zeros((B, kv // 16), dtype=torch.int32, device="cuda")
    with pytest.raises(qd.QdError) as ei:
        qd.attn_decode_noalloc(q, k, k, lens, kv, nkv, 0.1, out, block_tables=tbl)
    assert ei.value.code == qd._native.QD_EUNSUPPORTED and "scratch" in str(ei.value)
    assert torch.isnan(out).all()   # nothing enqueued
