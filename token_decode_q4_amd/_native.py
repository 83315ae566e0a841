"""ctypes binding of ``libqd.so`` (the C ABI declared in ``include/qd.h``).

Argument marshalling only: every step of the decode path runs in the HIP
library.  Device buffers are torch tensors on ``cuda`` (ROCm), streams are
torch streams; host arrays are numpy arrays.  If the library has not been
built this module raises on first use: there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqd.so")

QD_OK, QD_EINVAL, QD_ERANGE, QD_ENOMEM, QD_EUNSUPPORTED, QD_EHIP = 0, -1, -2, -3, -4, -5

# every function declared in include/qd.h
EXPORTS = ("qd_create", "qd_create_batch", "qd_set_prompt_seq", "qd_generate_batch", "qd_decode_step_batch",
           "qd_destroy", "qd_decode_step", "qd_set_prompt", "qd_generate", "qd_prefill", "qd_prefill_chunk",
           "qd_gemv_q4_0", "qd_gemv_q4_0_batch", "qd_gemv_q4_0_experts", "qd_rope_inv_freq", "qd_attn_workspace_bytes",
           "qd_attn_decode_kv8", "qd_attn_decode", "qd_attn_noalloc_max_bytes", "qd_attn_decode_noalloc",
           "qd_check",
           "qd_stream_read_groups", "qd_stream_read", "qd_last_error")


class QdError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"qd error {code}: {msg}")
        self.code = code


class Q4(C.Structure):
    _fields_ = [("d", C.c_void_p), ("qs", C.c_void_p), ("rows", C.c_int32), ("cols", C.c_int32)]


class LayerWeights(C.Structure):
    _fields_ = [("attn_norm", C.c_void_p), ("ffn_norm", C.c_void_p), ("q_norm", C.c_void_p),
                ("k_norm", C.c_void_p)] + [(n, Q4) for n in
                                           ("wq", "wk", "wv", "wo", "wgate", "wup", "wdown",
                                            "attn_gate")]


class Weights(C.Structure):
    _fields_ = [("embed", Q4), ("lm_head", Q4), ("final_norm", C.c_void_p),
                ("layers", C.POINTER(LayerWeights))]


class Config(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("layers", C.c_int32), ("n_heads", C.c_int32),
                ("n_kv", C.c_int32), ("head_dim", C.c_int32), ("intermediate", C.c_int32),
                ("vocab", C.c_int32), ("eps", C.c_float), ("rot_dim", C.c_int32),
                ("inv_freq", C.c_void_p), ("tied", C.c_int32), ("qk_norm", C.c_int32),
                ("max_seq", C.c_int32), ("kv_paged", C.c_int32), ("kv_block_size", C.c_int32),
                ("num_kv_blocks", C.c_int32), ("block_table", C.c_void_p),
                ("use_graph", C.c_int32), ("layer_kernel", C.c_int32),
                ("kv_fp8", C.c_int32), ("k_scale", C.c_float), ("v_scale", C.c_float),
                ("attn_out_gate", C.c_int32)]


class AttnArgs(C.Structure):
    _fields_ = [("q", C.c_void_p), ("k", C.c_void_p), ("v", C.c_void_p),
                ("block_tables", C.c_void_p), ("max_blocks_per_seq", C.c_int32),
                ("block_size", C.c_int32), ("kv_lens", C.c_void_p), ("max_kv_len", C.c_int32),
                ("B", C.c_int32), ("nq", C.c_int32), ("nkv", C.c_int32), ("head_dim", C.c_int32),
                ("scale", C.c_float), ("out", C.c_void_p)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run python token_decode_q4_amd/build.py")
        # torch first: its HIP runtime carries the same soname as the one the
        # library links (libamdhip64.so.7), so the library binds to it and the
        # process holds one HIP runtime, the one that owns the tensors passed
        # in.  (Loaded on its own inside a process that later imports torch,
        # the library's runtime has reported no device at its first call.)
        import torch  # noqa: F401
        L = C.CDLL(LIB_PATH)
        L.qd_create.argtypes = [C.POINTER(Config), C.POINTER(Weights), C.c_void_p,
                                C.POINTER(C.c_void_p)]
        L.qd_destroy.argtypes = [C.c_void_p]
        L.qd_decode_step.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p,
                                     C.c_void_p]
        L.qd_set_prompt.argtypes = [C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p]
        L.qd_generate.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p,
                                  C.c_void_p]
        L.qd_prefill.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p]
        L.qd_prefill_chunk.argtypes = []
        L.qd_prefill_chunk.restype = C.c_int32
        L.qd_gemv_q4_0.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32,
                                   C.c_int32, C.c_void_p]
        L.qd_gemv_q4_0_batch.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32,
                                         C.c_int32, C.c_int32, C.c_void_p]
        L.qd_gemv_q4_0_experts.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_int32,
                                           C.c_void_p, C.c_void_p, C.c_int32, C.c_int32, C.c_void_p]
        L.qd_rope_inv_freq.argtypes = [C.c_float, C.c_int32, C.c_int32, C.c_float, C.c_float,
                                       C.c_float, C.c_float, C.c_void_p]
        L.qd_attn_workspace_bytes.restype = C.c_size_t
        L.qd_attn_workspace_bytes.argtypes = [C.c_int32] * 5
        L.qd_attn_decode.argtypes = [C.POINTER(AttnArgs), C.c_void_p, C.c_size_t, C.c_void_p]
        L.qd_attn_decode_kv8.argtypes = [C.POINTER(AttnArgs), C.c_float, C.c_float, C.c_void_p,
                                         C.c_size_t, C.c_void_p]
        L.qd_attn_noalloc_max_bytes.restype = C.c_size_t
        L.qd_attn_noalloc_max_bytes.argtypes = []
        L.qd_attn_decode_noalloc.restype = C.c_int
        L.qd_attn_decode_noalloc.argtypes = [C.POINTER(AttnArgs), C.c_void_p]
        L.qd_check.argtypes = [C.c_void_p, C.c_void_p]
        L.qd_stream_read_groups.restype = C.c_size_t
        L.qd_stream_read_groups.argtypes = [C.c_size_t]
        L.qd_stream_read.argtypes = [C.c_void_p, C.c_size_t, C.c_void_p, C.c_void_p]
        L.qd_last_error.restype = C.c_char_p
        L.qd_create_batch.argtypes = [C.POINTER(Config), C.POINTER(Weights), C.c_int32, C.c_void_p,
                                      C.POINTER(C.c_void_p)]
        L.qd_set_prompt_seq.argtypes = [C.c_void_p, C.c_int32, C.c_void_p, C.c_int32, C.c_void_p]
        L.qd_generate_batch.argtypes = [C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p,
                                        C.c_void_p]
        L.qd_decode_step_batch.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                           C.c_void_p]
        for n in ("qd_create_batch", "qd_set_prompt_seq", "qd_generate_batch", "qd_decode_step_batch"):
            getattr(L, n).restype = C.c_int
        for n in ("qd_create", "qd_destroy", "qd_decode_step", "qd_set_prompt", "qd_generate", "qd_prefill",
                  "qd_gemv_q4_0", "qd_attn_decode", "qd_check", "qd_stream_read"):
            getattr(L, n).restype = C.c_int
        _lib = L
    return _lib


def check(rc: int):
    if rc != QD_OK:
        raise QdError(rc, lib().qd_last_error().decode())
    return rc


def _ptr(t) -> int | None:
    """Device pointer of a torch tensor (or None)."""
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


# ----------------------------------------------------------------- standalone ops

def gemv_q4_0(d, qs, x, y, stream=None) -> int:
    """y[N] = W x on the device; d uint16/int16 [N, K/32], qs uint8 [N, K/32, 16]."""
    N = d.shape[0]
    K = x.shape[0]
    return check(lib().qd_gemv_q4_0(_ptr(d), _ptr(qs), _ptr(x), _ptr(y), N, K, _stream(stream)))


def gemv_q4_0_batch(d, qs, x, y, stream=None) -> int:
    """Y[b] = W X[b]: x device f32 [B][K], y device f32 [B][N] (both contiguous)."""
    B, K = x.shape
    N = y.shape[1]
    return check(lib().qd_gemv_q4_0_batch(_ptr(d), _ptr(qs), _ptr(x), _ptr(y), N, K, B,
                                          _stream(stream)))


def gemv_q4_0_experts(d, qs, experts, x, y, stream=None) -> int:
    """y[j] = W[experts[j]] x: d [E, N, K/32] uint16/int16, qs [E, N, K/32, 16] uint8,
    experts device int32 [k], x device f32 [K], y device f32 [k, N]."""
    E, N = d.shape[0], d.shape[1]
    K = x.shape[0]
    k = experts.shape[0]
    return check(lib().qd_gemv_q4_0_experts(_ptr(d), _ptr(qs), _ptr(experts), E, k, _ptr(x),
                                            _ptr(y), N, K, _stream(stream)))


ROPE_SCALING = {"default": 0, "linear": 1, "llama3": 2}


def rope_inv_freq(theta: float, rot_dim: int, scaling: str = "default", factor: float = 1.0,
                  low_freq_factor: float = 1.0, high_freq_factor: float = 4.0,
                  original_max_pos: float = 8192.0) -> np.ndarray:
    """f32 [rot_dim/2] rotary frequencies from the library (qd_rope_inv_freq)."""
    if scaling not in ROPE_SCALING:
        raise QdError(QD_EUNSUPPORTED, f"rotary scaling type {scaling!r} is not implemented")
    out = np.empty(max(0, rot_dim // 2), dtype=np.float32)
    check(lib().qd_rope_inv_freq(theta, rot_dim, ROPE_SCALING[scaling], factor, low_freq_factor,
                                 high_freq_factor, original_max_pos, out.ctypes.data))
    return out


def stream_read_groups(nbytes: int) -> int:
    return int(lib().qd_stream_read_groups(nbytes))


def prefill_chunk() -> int:
    """Prompt positions per qd_prefill chunk (qd_prefill_chunk)."""
    return int(lib().qd_prefill_chunk())


def stream_read(src, sink, nbytes=None, stream=None) -> int:
    """Streaming read of the device tensor src (all of it, or its first nbytes):
    sink (device int32/uint32, stream_read_groups(nbytes) words) gets one XOR per
    workgroup."""
    n = src.numel() * src.element_size() if nbytes is None else int(nbytes)
    return check(lib().qd_stream_read(_ptr(src), n, _ptr(sink), _stream(stream)))


def attn_workspace_bytes(B, nq, nkv, head_dim, max_kv_len) -> int:
    return int(lib().qd_attn_workspace_bytes(B, nq, nkv, head_dim, max_kv_len))


def attn_decode(q, k, v, kv_lens, max_kv_len, nkv, scale, out, workspace, block_tables=None,
                block_size=16, stream=None) -> int:
    B, nq, hd = q.shape
    a = AttnArgs(_ptr(q), _ptr(k), _ptr(v), _ptr(block_tables),
                 0 if block_tables is None else block_tables.shape[1], block_size, _ptr(kv_lens),
                 int(max_kv_len), B, nq, nkv, hd, float(scale), _ptr(out))
    return check(lib().qd_attn_decode(C.byref(a), _ptr(workspace), workspace.numel() *
                                      workspace.element_size(), _stream(stream)))


def attn_noalloc_max_bytes() -> int:
    return int(lib().qd_attn_noalloc_max_bytes())


def attn_decode_noalloc(q, k, v, kv_lens, max_kv_len, nkv, scale, out, block_tables=None,
                        block_size=16, stream=None) -> int:
    """attn_decode with its split partials in the library's per-GPU scratch
    array (no workspace argument, no allocation)."""
    B, nq, hd = q.shape
    a = AttnArgs(_ptr(q), _ptr(k), _ptr(v), _ptr(block_tables),
                 0 if block_tables is None else block_tables.shape[1], block_size, _ptr(kv_lens),
                 int(max_kv_len), B, nq, nkv, hd, float(scale), _ptr(out))
    return check(lib().qd_attn_decode_noalloc(C.byref(a), _stream(stream)))


def attn_decode_kv8(q, k8, v8, kv_lens, max_kv_len, nkv, scale, k_scale, v_scale, out, workspace,
                    block_tables=None, block_size=16, stream=None) -> int:
    """attn_decode over an fp8 e4m3 cache: k8 / v8 device uint8 pools (same
    layouts as the f16 ones), element = e4m3 value * k_scale (K) or * v_scale (V)."""
    B, nq, hd = q.shape
    a = AttnArgs(_ptr(q), _ptr(k8), _ptr(v8), _ptr(block_tables),
                 0 if block_tables is None else block_tables.shape[1], block_size, _ptr(kv_lens),
                 int(max_kv_len), B, nq, nkv, hd, float(scale), _ptr(out))
    return check(lib().qd_attn_decode_kv8(C.byref(a), float(k_scale), float(v_scale), _ptr(workspace),
                                          workspace.numel() * workspace.element_size(),
                                          _stream(stream)))


# ----------------------------------------------------------------- model

def _q4(W) -> Q4:
    return Q4(W.d.ctypes.data, W.qs.ctypes.data, W.rows, W.cols)


class Model:
    """A decode model built from host q4_0 weights (``synth.ModelInputs``-like)."""

    def __init__(self, mi, use_graph: bool = True, stream=None, paged: bool | None = None,
                 max_seq: int | None = None, num_kv_blocks: int | None = None,
                 layer_kernel: bool = False, kv_fp8: bool = False, k_scale: float = 1.0,
                 v_scale: float = 1.0, batch: int = 1, block_table=None):
        """batch > 1: a batched model of that many sequences (qd_create_batch);
        block_table (paged) then holds batch tables of ceil(max_seq/16) entries
        (None: the identity)."""
        s = mi.shape
        self.batch = int(batch)
        self.shape = s
        self.vocab = s.vocab
        self.max_seq = max_seq or s.max_seq
        paged = s.kv_paged if paged is None else paged
        keep = []
        layers = (LayerWeights * s.layers)()
        gated = getattr(mi.layers[0], "attn_gate", None) is not None
        for i, L in enumerate(mi.layers):
            ns = [np.ascontiguousarray(a, dtype=np.float32) for a in
                  (L.attn_norm, L.ffn_norm, L.q_norm, L.k_norm)]
            keep.append(ns)
            ag = _q4(L.attn_gate) if gated else Q4(None, None, 0, 0)
            layers[i] = LayerWeights(*[a.ctypes.data for a in ns],
                                     *[_q4(m) for m in (L.wq, L.wk, L.wv, L.wo, L.wgate, L.wup,
                                                        L.wdown)], ag)
        fn = np.ascontiguousarray(mi.final_norm, dtype=np.float32)
        inv = np.ascontiguousarray(mi.inv_freq, dtype=np.float32)
        nblk_need = (self.max_seq + 15) // 16
        table = None
        if paged:
            if block_table is not None:
                table = np.ascontiguousarray(block_table, dtype=np.int32).ravel()
            elif self.batch == 1 and len(mi.block_table) >= nblk_need:
                table = np.ascontiguousarray(mi.block_table[:nblk_need], dtype=np.int32)
            need = nblk_need * self.batch
            nblocks = num_kv_blocks or (max(int(table.max()) + 1, need) if table is not None else need)
        else:
            nblocks = 0
        w = Weights(_q4(mi.embed), _q4(mi.lm_head), fn.ctypes.data, layers)
        cfg = Config(s.hidden, s.layers, s.n_heads, s.n_kv, s.head_dim, s.intermediate, s.vocab,
                     float(s.eps), s.rot_dim, inv.ctypes.data, int(s.tied), int(s.qk_norm),
                     self.max_seq, int(bool(paged)), 16, nblocks,
                     None if table is None else table.ctypes.data, int(bool(use_graph)),
                     int(bool(layer_kernel)), int(bool(kv_fp8)), float(k_scale), float(v_scale),
                     int(gated))
        h = C.c_void_p()
        if self.batch == 1:
            check(lib().qd_create(C.byref(cfg), C.byref(w), _stream(stream), C.byref(h)))
        else:
            check(lib().qd_create_batch(C.byref(cfg), C.byref(w), self.batch, _stream(stream), C.byref(h)))
        self._h = h
        del keep

    # batched model (batch > 1)
    def set_prompt_seq(self, seq: int, tokens, stream=None):
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        return check(lib().qd_set_prompt_seq(self._h, int(seq), t.ctypes.data, t.size, _stream(stream)))

    def generate_batch(self, pos0, n_steps: int, tokens=None, logits_last=None, stream=None):
        """Every sequence b runs positions pos0[b] .. pos0[b]+n_steps-1;
        tokens: device int32 [batch, n_steps]; logits_last: device f32 [batch, vocab]."""
        p = np.ascontiguousarray(pos0, dtype=np.int32)
        return check(lib().qd_generate_batch(self._h, p.ctypes.data, int(n_steps), _ptr(tokens),
                                             _ptr(logits_last), _stream(stream)))

    def decode_step_batch(self, tokens, pos, logits=None, next_tok=None, stream=None):
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        p = np.ascontiguousarray(pos, dtype=np.int32)
        return check(lib().qd_decode_step_batch(self._h, t.ctypes.data, p.ctypes.data, _ptr(logits),
                                                _ptr(next_tok), _stream(stream)))

    def decode_step(self, token: int, pos: int, logits=None, next_tok=None, stream=None):
        return check(lib().qd_decode_step(self._h, int(token), int(pos), _ptr(logits),
                                          _ptr(next_tok), _stream(stream)))

    def set_prompt(self, tokens, stream=None):
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        return check(lib().qd_set_prompt(self._h, t.ctypes.data, t.size, _stream(stream)))

    def generate(self, pos0: int, n_steps: int, tokens=None, logits_last=None, stream=None):
        return check(lib().qd_generate(self._h, int(pos0), int(n_steps), _ptr(tokens),
                                       _ptr(logits_last), _stream(stream)))

    def prefill(self, pos0: int, n: int, logits_last=None, stream=None):
        """Chunked prefill of positions pos0 .. pos0+n-1 (qd_prefill)."""
        return check(lib().qd_prefill(self._h, int(pos0), int(n), _ptr(logits_last), _stream(stream)))

    def check(self, stream=None):
        """Synchronise and raise QdError if the device recorded an error since
        the last check (qd_check)."""
        return check(lib().qd_check(self._h, _stream(stream)))

    def close(self):
        if getattr(self, "_h", None):
            lib().qd_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
