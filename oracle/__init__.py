"""Python face of the f64 CPU oracle (``qd_oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline use this package; the product path never imports it.  It shares no
code with the HIP library; the only common module is ``synth`` (seeded input
generation, no decode arithmetic).
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import build as _build

_lib = None


class _Q4(C.Structure):
    _fields_ = [("d", C.c_void_p), ("qs", C.c_void_p), ("rows", C.c_int64), ("cols", C.c_int64)]


class _Layer(C.Structure):
    _fields_ = [("attn_norm", C.c_void_p), ("ffn_norm", C.c_void_p), ("q_norm", C.c_void_p),
                ("k_norm", C.c_void_p)] + [(n, _Q4) for n in
                                           ("wq", "wk", "wv", "wo", "wgate", "wup", "wdown",
                                            "wag")]


class _Cfg(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("hidden", "layers", "n_heads", "n_kv", "head_dim",
                                         "intermediate", "vocab", "rot_dim", "qk_norm",
                                         "max_seq", "kv_round")] + \
               [("eps", C.c_double), ("inv_freq", C.c_void_p), ("k_scale", C.c_double),
                ("v_scale", C.c_double), ("attn_out_gate", C.c_int32)]


def lib():
    global _lib
    if _lib is None:
        # QD_ORACLE_LIB points the wrapper at another build of qd_oracle.c
        # (the mutation test uses it to load deliberately broken copies)
        path = os.environ.get("QD_ORACLE_LIB") or _build.LIB
        if path == _build.LIB and not os.path.exists(path):
            _build.build()
        L = C.CDLL(path)
        L.or_f16_to_f64.restype = C.c_double
        L.or_f16_to_f64.argtypes = [C.c_uint16]
        L.or_f64_to_f16.restype = C.c_uint16
        L.or_f64_to_f16.argtypes = [C.c_double]
        L.or_e4m3_to_f64.restype = C.c_double
        L.or_e4m3_to_f64.argtypes = [C.c_uint8]
        L.or_f64_to_e4m3.restype = C.c_uint8
        L.or_f64_to_e4m3.argtypes = [C.c_double]
        L.or_dequant_q4_0.argtypes = [C.POINTER(_Q4), C.c_void_p]
        L.or_gemv_q4_0.argtypes = [C.POINTER(_Q4), C.c_void_p, C.c_void_p, C.c_int]
        L.or_rmsnorm.argtypes = [C.c_void_p, C.c_void_p, C.c_int64, C.c_double, C.c_void_p]
        L.or_rope_neox.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_void_p, C.c_int64]
        L.or_attn_decode.restype = C.c_int
        L.or_attn_decode.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32,
                                     C.c_int32, C.c_int32, C.c_void_p, C.c_int32, C.c_int32,
                                     C.c_int32, C.c_int32, C.c_double, C.c_void_p, C.c_int]
        L.or_model_create.restype = C.c_void_p
        L.or_model_create.argtypes = [C.POINTER(_Cfg), C.POINTER(_Q4), C.c_void_p, C.c_void_p,
                                      C.POINTER(_Q4), C.c_int]
        L.or_model_step.restype = C.c_int
        L.or_model_step.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_void_p]
        L.or_model_kv.restype = C.c_int
        L.or_model_kv.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                  C.c_void_p]
        L.or_model_load_kv.restype = C.c_int
        L.or_model_load_kv.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_void_p,
                                       C.c_void_p]
        L.or_model_destroy.argtypes = [C.c_void_p]
        _lib = L
    return _lib


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _p(a: np.ndarray) -> int:
    return a.ctypes.data


def _q4(W) -> _Q4:
    d = np.ascontiguousarray(W.d, dtype=np.uint16)
    qs = np.ascontiguousarray(W.qs, dtype=np.uint8)
    assert d.shape[0] == qs.shape[0] and d.shape[1] == qs.shape[1] and qs.shape[2] == 16
    s = _Q4(_p(d), _p(qs), d.shape[0], d.shape[1] * 32)
    s._keep = (d, qs)
    return s


# --------------------------------------------------------------------------- primitives

def f16_to_f64(bits) -> np.ndarray:
    L = lib()
    b = np.asarray(bits, dtype=np.uint16)
    return np.array([L.or_f16_to_f64(int(x)) for x in b.ravel()], dtype=np.float64).reshape(b.shape)


def f64_to_f16(vals) -> np.ndarray:
    L = lib()
    v = np.asarray(vals, dtype=np.float64)
    return np.array([L.or_f64_to_f16(float(x)) for x in v.ravel()], dtype=np.uint16).reshape(v.shape)


def dequant(W) -> np.ndarray:
    q = _q4(W)
    out = np.empty((q.rows, q.cols), dtype=np.float64)
    lib().or_dequant_q4_0(C.byref(q), _p(out))
    return out


def gemv(W, x, nthreads: int | None = None) -> np.ndarray:
    """y = dequant(W) @ x in f64 (x is promoted exactly from its dtype)."""
    q = _q4(W)
    xx = np.ascontiguousarray(x, dtype=np.float64)
    assert xx.shape == (q.cols,)
    y = np.empty(q.rows, dtype=np.float64)
    lib().or_gemv_q4_0(C.byref(q), _p(xx), _p(y), nthreads or default_threads())
    return y


def rmsnorm(x, w, eps: float) -> np.ndarray:
    xx = np.ascontiguousarray(x, dtype=np.float64)
    ww = np.ascontiguousarray(w, dtype=np.float32)
    out = np.empty_like(xx)
    lib().or_rmsnorm(_p(xx), _p(ww), xx.size, float(eps), _p(out))
    return out


def rope(v, rot: int, inv_freq, pos: int) -> np.ndarray:
    vv = np.array(v, dtype=np.float64, copy=True)
    f = np.ascontiguousarray(inv_freq, dtype=np.float32)
    assert f.size >= rot // 2
    lib().or_rope_neox(_p(vv), vv.size, int(rot), _p(f), int(pos))
    return vv


def rope_inv_freq(theta: float, rot_dim: int, scaling: str = "default", factor: float = 1.0,
                  low_freq_factor: float = 1.0, high_freq_factor: float = 4.0,
                  original_max_pos: float = 8192.0) -> np.ndarray:
    """Rotary frequencies with rotary scaling, in f64 (inferencelayer cuda_llm.rs
    page, Cfg::rope_inv_freq; the exponent over rot_dim as in the partial-rotary
    reading): base f_i = theta^(-2i/rot_dim).  "linear": every f_i / factor.
    "llama3": with wavelength w_i = 2 pi / f_i, low = orig / low_freq_factor and
    high = orig / high_freq_factor: w_i > low -> f_i / factor; high <= w_i <= low
    -> (1 - s) f_i / factor + s f_i with s = (orig / w_i - low_freq_factor) /
    (high_freq_factor - low_freq_factor); w_i < high -> f_i.  Other types are
    refused (ValueError)."""
    out = []
    for i in range(rot_dim // 2):
        f = float(theta) ** (-(2.0 * i) / float(rot_dim))
        if scaling == "default":
            pass
        elif scaling == "linear":
            f = f / factor
        elif scaling == "llama3":
            wavelength = 2.0 * np.pi / f
            low_wl = original_max_pos / low_freq_factor
            high_wl = original_max_pos / high_freq_factor
            if wavelength > low_wl:
                f = f / factor
            elif wavelength >= high_wl:
                s = (original_max_pos / wavelength - low_freq_factor) / (high_freq_factor - low_freq_factor)
                f = (1.0 - s) * (f / factor) + s * f
        else:
            raise ValueError(f"rotary scaling type {scaling!r} is not implemented")
        out.append(f)
    return np.array(out, dtype=np.float64)


def f64_to_e4m3(vals) -> np.ndarray:
    """fp8 e4m3 codes of f64 values (qd_oracle.c or_f64_to_e4m3: round to
    nearest even, saturating at +-448)."""
    L = lib()
    v = np.asarray(vals, dtype=np.float64)
    return np.array([L.or_f64_to_e4m3(float(x)) for x in v.ravel()], dtype=np.uint8).reshape(v.shape)


def e4m3_to_f64_c(codes) -> np.ndarray:
    """qd_oracle.c's own e4m3 decode (the one its model uses)."""
    L = lib()
    c = np.asarray(codes, dtype=np.uint8)
    return np.array([L.or_e4m3_to_f64(int(x)) for x in c.ravel()], dtype=np.float64).reshape(c.shape)


def e4m3_to_f64(codes) -> np.ndarray:
    """Exact values of OCP fp8 e4m3 codes (the fp8 KV cache): sign bit 7,
    exponent bits 6..3 with bias 7, mantissa bits 2..0; exponent 0 is
    subnormal (m * 2^-9); 0x7f and 0xff are NaN; there is no infinity."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    val = np.where(c >> 7, -mag, mag)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


def attn_decode_e4m3(q, k8, v8, kv_lens, nkv: int, scale: float, k_scale: float, v_scale: float,
                     block_tables=None, block_size: int = 16, contig_max_kv: int = 0,
                     nthreads: int | None = None) -> np.ndarray:
    """The attention of attn_decode over an fp8 e4m3 cache: K = e4m3(k8) *
    k_scale, V = e4m3(v8) * v_scale.  Every e4m3 value is an f16 value, so the
    decoded caches go to attn_decode as f16 bits unchanged; k_scale multiplies
    every score (folded into the softmax scale) and v_scale every output."""
    kv = e4m3_to_f64(k8)
    vv = e4m3_to_f64(v8)
    if np.isnan(kv).any() or np.isnan(vv).any():
        raise ValueError("NaN code in the cache")
    # exact (no rounding happens), checked on every element
    kb = kv.astype(np.float16).view(np.uint16)
    vb = vv.astype(np.float16).view(np.uint16)
    if not (np.array_equal(kb.view(np.float16).astype(np.float64), kv)
            and np.array_equal(vb.view(np.float16).astype(np.float64), vv)):
        raise AssertionError("an e4m3 value was not exact in f16")
    out = attn_decode(q, kb, vb, kv_lens, nkv, float(scale) * float(k_scale), block_tables,
                      block_size, contig_max_kv, nthreads)
    return out * float(v_scale)


def attn_decode(q, k, v, kv_lens, nkv: int, scale: float, block_tables=None,
                block_size: int = 16, contig_max_kv: int = 0,
                nthreads: int | None = None) -> np.ndarray:
    """Decode attention; see or_attn_decode.  q f32 [B, nq, hd]."""
    qq = np.ascontiguousarray(q, dtype=np.float32)
    B, nq, hd = qq.shape
    kk = np.ascontiguousarray(k, dtype=np.uint16)
    vv = np.ascontiguousarray(v, dtype=np.uint16)
    lens = np.ascontiguousarray(kv_lens, dtype=np.int32)
    out = np.empty((B, nq, hd), dtype=np.float64)
    if block_tables is not None:
        bt = np.ascontiguousarray(block_tables, dtype=np.int32)
        tp, mbps = _p(bt), bt.shape[1]
    else:
        bt, tp, mbps = None, None, 0
    rc = lib().or_attn_decode(_p(qq), _p(kk), _p(vv), tp, mbps, block_size, contig_max_kv,
                              _p(lens), B, nq, nkv, hd, float(scale), _p(out),
                              nthreads or default_threads())
    if rc != 0:
        raise ValueError("or_attn_decode rejected its arguments")
    return out


def attn_inputs(a, nthreads: int | None = None) -> np.ndarray:
    """Oracle attention for a ``synth.AttnInputs`` (paged)."""
    return attn_decode(a.q, a.k_pool, a.v_pool, a.kv_lens, a.nkv, 1.0 / np.sqrt(a.hd),
                       block_tables=a.block_tables, block_size=a.block, nthreads=nthreads)


# --------------------------------------------------------------------------- model

class Model:
    """The oracle decoder over a ``synth.ModelInputs``; KV cache kept inside."""

    def __init__(self, mi, nthreads: int | None = None, kv_round: bool = True,
                 kv_fp8: bool = False, k_scale: float = 1.0, v_scale: float = 1.0):
        """kv_round: K/V stored as binary16 (the method) or kept in f64 (for
        pins); kv_fp8: stored as fp8 e4m3 of value / k_scale (K) and value /
        v_scale (V) instead."""
        s = mi.shape
        self.mi = mi
        self.vocab = s.vocab
        self._embed = _q4(mi.embed)
        self._lm = _q4(mi.lm_head)
        self._keep = []
        layers = (_Layer * s.layers)()
        for i, Lw in enumerate(mi.layers):
            ns = [np.ascontiguousarray(a, dtype=np.float32) for a in
                  (Lw.attn_norm, Lw.ffn_norm, Lw.q_norm, Lw.k_norm)]
            qs = [_q4(m) for m in (Lw.wq, Lw.wk, Lw.wv, Lw.wo, Lw.wgate, Lw.wup, Lw.wdown)]
            ag = getattr(Lw, "attn_gate", None)
            qs.append(_q4(ag) if ag is not None else _Q4(None, None, 0, 0))
            self._keep.append((ns, qs))
            layers[i] = _Layer(_p(ns[0]), _p(ns[1]), _p(ns[2]), _p(ns[3]), *qs)
        self._layers = layers
        self._final = np.ascontiguousarray(mi.final_norm, dtype=np.float32)
        self._inv = np.ascontiguousarray(mi.inv_freq, dtype=np.float32)
        self._cfg = _Cfg(s.hidden, s.layers, s.n_heads, s.n_kv, s.head_dim, s.intermediate,
                         s.vocab, s.rot_dim, int(s.qk_norm), s.max_seq,
                         2 if kv_fp8 else int(kv_round), float(s.eps), _p(self._inv),
                         float(k_scale), float(v_scale),
                         int(getattr(mi.layers[0], "attn_gate", None) is not None))
        self.nthreads = nthreads or default_threads()
        h = lib().or_model_create(C.byref(self._cfg), C.byref(self._embed), self._layers,
                                  _p(self._final), C.byref(self._lm), self.nthreads)
        if not h:
            raise ValueError("oracle rejected the model configuration")
        self._h = h

    def step(self, token: int, pos: int) -> np.ndarray:
        out = np.empty(self.vocab, dtype=np.float64)
        if lib().or_model_step(self._h, int(token), int(pos), _p(out)) != 0:
            raise ValueError(f"oracle step rejected token={token} pos={pos}")
        return out

    def kv(self, layer: int, pos: int, kv_head: int, which_v: bool) -> np.ndarray:
        out = np.empty(self.mi.shape.head_dim, dtype=np.float64)
        if lib().or_model_kv(self._h, layer, pos, kv_head, int(which_v), _p(out)) != 0:
            raise ValueError("bad kv index")
        return out

    def load_kv(self, layer: int, pos0: int, k, v):
        """Store k, v [n, n_kv*head_dim] as the K/V of one layer at positions
        pos0 .. pos0+n-1 (no arithmetic; for timing steps at a long context)."""
        kk = np.ascontiguousarray(k, dtype=np.float64)
        vv = np.ascontiguousarray(v, dtype=np.float64)
        s = self.mi.shape
        assert kk.shape == vv.shape and kk.ndim == 2 and kk.shape[1] == s.n_kv * s.head_dim
        if lib().or_model_load_kv(self._h, int(layer), int(pos0), kk.shape[0], _p(kk), _p(vv)) != 0:
            raise ValueError("bad kv range")

    def close(self):
        if getattr(self, "_h", None):
            lib().or_model_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # interpreter shutdown
            pass


def greedy_pick(logits: np.ndarray):
    """Greedy choice over logits rounded to f32 (the precision the device
    compares in); lowest index wins ties.  Returns (token, top1 - top2 margin
    of the f64 logits)."""
    f32 = logits.astype(np.float32)
    tok = int(np.argmax(f32))
    top2 = np.partition(logits, -2)[-2:]
    return tok, float(top2[1] - top2[0])


def generate(model: Model, prompt, G: int, keep_logits_at=(), on_step=None):
    """Sequential-decode prefill of ``prompt`` (positions 0..P-1) then G greedy
    tokens: the logits at position P-1 give token 0, token i is fed at P+i-1.
    Returns (tokens[G], margins[G], {greedy index: logits f64})."""
    prompt = [int(t) for t in prompt]
    P = len(prompt)
    toks, margins, kept = [], [], {}
    keep = set(keep_logits_at)
    cur = prompt[0]
    for pos in range(P + G - 1):
        lg = model.step(cur, pos)
        if on_step is not None:
            on_step(pos)
        if pos + 1 < P:
            cur = prompt[pos + 1]
            continue
        gi = pos - (P - 1)
        t, mg = greedy_pick(lg)
        toks.append(t)
        margins.append(mg)
        if gi in keep:
            kept[gi] = lg.copy()
        cur = t
    return np.array(toks, dtype=np.int32), np.array(margins), kept
