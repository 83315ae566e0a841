"""q4_0 GEMV through the C ABI (qd_gemv_q4_0, qd_gemv_q4_0_batch) against the f64 oracle."""
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


def _gemv_batch(W, X):
    import torch
    import token_decode_q4_amd as qd
    Y = torch.full((X.shape[0], W.rows), float("nan"), dtype=torch.float32, device="cuda")
    qd.gemv_q4_0_batch(dev(W.d), dev(W.qs), dev(X), Y)
    return host(Y)


# Batched bar: normwise 1e-5.  From 6 vectors the matrix-core kernel runs (f16
# hi + lo operands, exact products, matrix-core f32 accumulation): measured
# 1.4e-6 .. 2.9e-6 against the f64 oracle, 0.3e-6 for the vector kernel; the
# GEMV bar itself is 1e-3.
BATCH_BAR = 1e-5


@pytest.mark.parametrize("idx", range(len(synth.GEMV_SHAPES)))
@pytest.mark.parametrize("B", [2, 5, 6, 8, 16])
def test_gemv_batch_sweep_shape(idx, B):
    """Y[b] = W X[b] at the sweep shapes, every column against the f64 oracle."""
    N, K = synth.GEMV_SHAPES[idx]
    say(f"gemv batch {B} x {N}x{K}")
    (W,), _ = synth.gemv_case(idx)
    X = synth.batch_x(7000 + idx, B, K)
    Y = _gemv_batch(W, X)
    assert np.all(np.isfinite(Y))
    for b in range(B):
        err = normwise(Y[b], oracle.gemv(W, X[b]))
        assert err <= BATCH_BAR, (b, err)


def _f32_bound(W, x):
    """Per-row scale of the f32 rounding error of the kernels' sum: the magnitudes
    the arithmetic handles, sum_j |w_j x_j| plus the -8 * d * sum(x) offset of
    every block (a forward error bound for a dot product is a small multiple of
    the unit roundoff times this)."""
    dense = oracle.dequant(W)
    d = np.abs(oracle.f16_to_f64(W.d))
    xa = np.abs(x.astype(np.float64))
    blk = xa.reshape(-1, 32).sum(axis=1)
    return np.abs(dense) @ xa + 8.0 * (d @ blk)


@pytest.mark.parametrize("B", [1, 2, 3, 4, 5, 6, 7, 8, 9, 11, 13, 16])
@pytest.mark.parametrize("N,K", [(1, 32), (17, 96), (100, 1024), (257, 3072), (4097, 2048),
                                 (70, 160), (1000, 4096), (65, 12288), (33, 1056)])
def test_gemv_batch_ragged(N, K, B):
    # below 6 vectors a batch with B * K above 32768 runs on the matrix cores
    W, _ = synth.random_gemv(2000 + N, N, K)
    X = synth.batch_x(3000 + N + B, B, K)
    Y = _gemv_batch(W, X)
    for b in range(B):
        # elementwise against the f32 error bound (a single short row can cancel
        # to far below its terms, where a relative bar would test rounding luck)
        err = np.abs(Y[b].astype(np.float64) - oracle.gemv(W, X[b]))
        assert np.all(err <= 1e-6 * _f32_bound(W, X[b])), b


@pytest.mark.parametrize("B", [3, 8, 16])
@pytest.mark.parametrize("x_scale", [1e-6, 1e-5, 1e5, 3e6])
def test_gemv_batch_input_scales(B, x_scale):
    """Inputs far from unit scale: 1e-5 and 1e-6 put an unscaled f16 lo half in
    the subnormal range, 1e5 and 3e6 overflow an unscaled f16 hi half.  The
    matrix-core kernel scales each vector chunk by a power of two first, so the
    normwise error stays at the unit-scale level (B = 3 at K = 12288 also runs
    on the matrix cores)."""
    for N, K in [(1000, 4096), (257, 12288)]:
        W, _ = synth.random_gemv(4100 + N, N, K)
        X = (synth.batch_x(4200 + B, B, K) * np.float32(x_scale)).astype(np.float32)
        X[0, 5] *= 64   # one large element in one chunk of the first vector
        Y = _gemv_batch(W, X)
        assert np.all(np.isfinite(Y))
        for b in range(B):
            err = normwise(Y[b], oracle.gemv(W, X[b]))
            assert err <= BATCH_BAR, (N, K, b, err)


def test_gemv_batch_equals_single_per_column():
    """Each column of the batch is the single-vector GEMV of that vector (to f32 rounding:
    the two kernels may sum in a different order)."""
    W, _ = synth.random_gemv(11, 6144, 4096)
    X = synth.batch_x(12, 8, 4096)
    Y = _gemv_batch(W, X)
    for b in range(8):
        y1 = _gemv(W, X[b])
        assert normwise(Y[b], y1.astype(np.float64)) <= BATCH_BAR


def test_gemv_batch_special_values():
    """Hand-built blocks, unit vectors in every column: exact."""
    K = 64
    codes = np.tile(np.arange(16, dtype=np.uint8), 8).reshape(2, 64)
    qs = (codes.reshape(2, 2, 32)[..., :16] | (codes.reshape(2, 2, 32)[..., 16:] << 4)).astype(np.uint8)
    d = np.array([[0x3C00, 0x3C00], [0xC000, 0x3C00]], dtype=np.uint16)
    W = synth.Q4Matrix(d, qs)
    dense = oracle.dequant(W)
    cols = [0, 1, 15, 16, 31, 32, 63, 40]
    X = np.zeros((len(cols), K), dtype=np.float32)
    for b, c in enumerate(cols):
        X[b, c] = 1.0
    Y = _gemv_batch(W, X)
    for b, c in enumerate(cols):
        assert np.array_equal(Y[b], dense[:, c].astype(np.float32)), b


def test_gemv_batch_k_zero_and_repeat():
    import ctypes as C
    import torch
    import token_decode_q4_amd as qd
    buf = torch.zeros(64, dtype=torch.float32, device="cuda")
    Y = torch.full((3, 300), float("nan"), dtype=torch.float32, device="cuda")
    p = C.c_void_p(buf.data_ptr())
    assert qd.lib().qd_gemv_q4_0_batch(p, p, p, C.c_void_p(Y.data_ptr()), 300, 0, 3, None) == 0
    assert np.array_equal(host(Y), np.zeros((3, 300), dtype=np.float32))
    W, _ = synth.random_gemv(5, 4096, 4096)
    X = synth.batch_x(6, 4, 4096)
    assert np.array_equal(_gemv_batch(W, X), _gemv_batch(W, X))


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


def test_gemv_batch_graph_replays_equal_eager():
    """qd_gemv_q4_0_batch captured in a graph (vector kernel at B = 3, matrix
    cores at B = 12), replayed several times with eager work and
    synchronisations between the replays: every replay equals the eager call."""
    import torch
    import token_decode_q4_amd as qd
    W, _ = synth.random_gemv(21, 4096, 2048)
    d, q = dev(W.d), dev(W.qs)
    for B in (3, 12):
        X = dev(synth.batch_x(22 + B, B, 2048))
        eager = torch.empty((B, 4096), dtype=torch.float32, device="cuda")
        qd.gemv_q4_0_batch(d, q, X, eager)
        torch.cuda.synchronize()
        ref = eager.cpu().numpy()
        Y = torch.full((B, 4096), float("nan"), dtype=torch.float32, device="cuda")
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            qd.gemv_q4_0_batch(d, q, X, Y, stream=s)   # warm-up outside the capture
            s.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                qd.gemv_q4_0_batch(d, q, X, Y, stream=s)
        for _ in range(3):
            Y.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert np.array_equal(Y.cpu().numpy(), ref)
            qd.gemv_q4_0_batch(d, q, X, eager)   # eager work between the replays
            torch.cuda.synchronize()



@pytest.mark.parametrize("N,K", [(1536, 2048), (100, 1024), (4097, 96)])
def test_gemv_experts_vs_oracle(N, K):
    """y[j] = W[experts[j]] x for picked experts (a repeat and the last expert
    included) against the f64 oracle of each expert's matrix; indices outside
    the stack give NaN rows and leave the other rows intact."""
    import torch
    import token_decode_q4_amd as qd
    E = 16
    W = synth.random_experts(900 + N, E, N, K)
    x = synth.batch_x(901, 1, K)[0]
    picks = np.array([3, 15, 0, 3, 9, -1, 7, 16], dtype=np.int32)
    y = torch.full((len(picks), N), 0.0, dtype=torch.float32, device="cuda")
    qd.gemv_q4_0_experts(dev(W.d.reshape(E, N, -1)), dev(W.qs.reshape(E, N, K // 32, 16)),
                         dev(picks), dev(x), y)
    got = host(y)
    for j, e in enumerate(picks):
        if 0 <= e < E:
            ref = oracle.gemv(synth.expert_rows(W, int(e), N), x)
            assert normwise(got[j], ref) <= 2e-6, (j, e)
        else:
            assert np.all(np.isnan(got[j])), (j, e)
    assert np.array_equal(got[0], got[3])   # the same expert twice: the same row, bitwise
