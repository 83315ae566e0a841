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


def test_gemv_k_zero_fills_zeros():
    """K = 0: y = 0 (a fill kernel; no memset node, so it stays capturable)."""
    import ctypes as C
    import torch
    import token_decode_q4_amd as qd
    say("gemv K=0")
    buf = torch.zeros(64, dtype=torch.float32, device="cuda")
    y = torch.full((300,), float("nan"), dtype=torch.float32, device="cuda")
    p = C.c_void_p(buf.data_ptr())
    assert qd.lib().qd_gemv_q4_0(p, p, p, C.c_void_p(y.data_ptr()), 300, 0, None) == 0
    assert np.array_equal(host(y), np.zeros(300, dtype=np.float32))


@pytest.mark.parametrize("nbytes", [16, 16 * 1023, 16 * 1024 + 48, 16 * 4096 * 3 + 16, 56737792])
def test_stream_read_xor(nbytes):
    """The streaming-read utility reads every word once: the XOR of its sink
    words equals the XOR of the buffer's 32-bit words (bit-exact)."""
    import torch
    import token_decode_q4_amd as qd
    say(f"stream read {nbytes} B")
    rng = np.random.default_rng(nbytes)
    words = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint32)
    src = torch.from_numpy(words.view(np.int32)).cuda()
    g = qd.stream_read_groups(nbytes)
    sink = torch.full((g,), -1, dtype=torch.int32, device="cuda")
    qd.stream_read(src, sink)
    got = np.bitwise_xor.reduce(host(sink).view(np.uint32))
    assert got == np.bitwise_xor.reduce(words)
