"""q4_0 GEMV through the C ABI (qd_gemv_q4_0) against the f64 oracle."""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import GEMV_BAR, dev, host, normwise, say

pytestmark = pytest.mark.gpu


def _gemv(W, x):
    import torch
    import token_decode_q4_amd as qd
    y = torch.full((W.rows,), float("nan"), dtype=torch.float32, device="cuda")
    qd.gemv_q4_0(dev(W.d), dev(W.qs), dev(x), y)
    return host(y)


@pytest.mark.parametrize("idx", range(len(synth.GEMV_SHAPES)))
def test_gemv_sweep_shape_full(idx):
    N, K = synth.GEMV_SHAPES[idx]
    say(f"gemv sweep shape {N}x{K}")
    (W,), x = synth.gemv_case(idx)
    ref = oracle.gemv(W, x)
    y = _gemv(W, x)
    err = normwise(y, ref)
    say(f"gemv {N}x{K}: normwise rel err {err:.3e}")
    assert np.all(np.isfinite(y))
    assert err <= GEMV_BAR
    # f32 arithmetic with an f64 reference stays far inside the bar
    assert err <= 2e-6


@pytest.mark.parametrize("N,K", [(1, 32), (5, 64), (17, 96), (33, 256), (100, 1024),
                                 (257, 3072), (1000, 4128), (31, 768), (4097, 2048),
                                 (3, 14144), (70, 160)])
def test_gemv_ragged(N, K):
    say(f"gemv ragged {N}x{K}")
    W, x = synth.random_gemv(1000 + N, N, K)
    ref = oracle.gemv(W, x)
    y = _gemv(W, x)
    assert normwise(y, ref) <= 2e-6


def test_gemv_special_values():
    """Hand-built blocks: every code, d = 1 and d = -2, x = unit vectors."""
    K = 64
    codes = np.tile(np.arange(16, dtype=np.uint8), 8).reshape(2, 64)
    qs = (codes.reshape(2, 2, 32)[..., :16] | (codes.reshape(2, 2, 32)[..., 16:] << 4)).astype(np.uint8)
    d = np.array([[0x3C00, 0x3C00], [0xC000, 0x3C00]], dtype=np.uint16)
    W = synth.Q4Matrix(d, qs)
    dense = oracle.dequant(W)
    for c in (0, 1, 15, 16, 31, 32, 63):
        x = np.zeros(K, dtype=np.float32)
        x[c] = 1.0
        assert np.array_equal(_gemv(W, x), dense[:, c].astype(np.float32))


def test_gemv_repeat_is_bitwise_stable():
    W, x = synth.random_gemv(5, 4096, 4096)
    a = _gemv(W, x)
    b = _gemv(W, x)
    assert np.array_equal(a, b)
