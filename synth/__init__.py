"""Seeded synthetic inputs for the batch-1 q4_0 decode path.

This module is the only code the CPU oracle (``oracle/``) and the HIP path
(``token_decode_q4_amd``) share.  It draws random numbers and lays them out in
the input formats the two sides consume; it holds none of the decode step's
arithmetic (no dequantisation, GEMV, norm, rotary, attention or softmax).

Formats produced (the interchange format both sides read):

* q4_0 matrix ``[rows, cols]`` as two arrays, row-major, blocks of 32 weights
  along a row (cols % 32 == 0):
    - ``d``  uint16 ``[rows, cols/32]``: IEEE binary16 bits of the block scale;
    - ``qs`` uint8  ``[rows, cols/32, 16]``: byte ``j`` of a block holds the
      code of element ``j`` in its low nibble and of element ``j+16`` in its
      high nibble.
  A weight's value is ``(code - 8) * d``.  (inferencelayer cuda_llm.rs page,
  ``Q4Dev``: one f16 scale and 16 bytes of nibbles per 32 weights; the nibble
  order inside a block is not shown on the pages, the low/high split is the
  reading chosen here.)
* f16 tensors as uint16 bit patterns.

Seeding: every tensor gets its own ``numpy.random.SeedSequence`` built from
``(config seed, tensor id, chunk id)``, so tensors can be drawn in parallel
and in any order with identical results.
"""
from __future__ import annotations

import concurrent.futures as _cf
import hashlib
import os
from dataclasses import dataclass, field

import numpy as np

WEIGHT_STD = 0.02      # weights ~ N(0, 0.02) before q4_0 quantisation (std, not variance)
NORM_STD = 0.1         # norm vectors ~ 1 + N(0, 0.1), kept f32
ROW_CHUNK_ELEMS = 1 << 23  # elements drawn per chunk of a large matrix


# --------------------------------------------------------------------------- configs

@dataclass(frozen=True)
class ModelShape:
    name: str
    seed: int
    layers: int
    hidden: int
    n_heads: int
    n_kv: int
    head_dim: int
    intermediate: int
    vocab: int
    tied: bool
    qk_norm: bool
    rope_theta: float
    rot_dim: int
    eps: float
    kv_paged: bool
    max_seq: int
    prompt_len: int
    gen: int
    kv_block_size: int = 16
    shuffle_blocks: bool = True


MODELS = {
    # tiny dense decoder: 2 layers, hidden 256, 4/2 heads of 64, SwiGLU 768,
    # vocab 1024, tied, contiguous KV; 16 prompt tokens + 32 greedy tokens
    "tiny": ModelShape("tiny", 1, 2, 256, 4, 2, 64, 768, 1024, True, True, 1e6, 64, 1e-6,
                       False, 48, 16, 32),
    # the tiny decoder with an LM head of its own (drawn from its own tensor
    # id; every other tensor equals the tiny one's)
    "tiny-untied": ModelShape("tiny-untied", 1, 2, 256, 4, 2, 64, 768, 1024, False, True, 1e6,
                              64, 1e-6, False, 48, 16, 32),
    # the tiny decoder with partial rotary: the first 32 of 64 dims of each
    # q/k head turn (inv_freq = 1e6^(-2i/32), 16 frequencies), the rest pass
    "tiny-rot32": ModelShape("tiny-rot32", 1, 2, 256, 4, 2, 64, 768, 1024, True, True, 1e6,
                             32, 1e-6, False, 48, 16, 32),
    # the tiny decoder at sizes that are not multiples of 256: hidden 288 and
    # SwiGLU 800 (9 and 25 q4_0 blocks per row, a ragged last chunk), vocab
    # 1000 (a ragged last row tile)
    "tiny-odd": ModelShape("tiny-odd", 7, 2, 288, 4, 2, 64, 800, 1000, True, True, 1e6, 64, 1e-6,
                           False, 48, 16, 32),
    # the tiny decoder with all 8 query heads on one kv head (GQA group 8)
    "tiny-gq8": ModelShape("tiny-gq8", 8, 2, 256, 8, 1, 64, 768, 1024, True, True, 1e6, 64, 1e-6,
                           False, 48, 16, 32),
    # the tiny decoder with a kv head per query head (GQA group 1)
    "tiny-mha": ModelShape("tiny-mha", 9, 2, 256, 4, 4, 64, 768, 1024, True, True, 1e6, 64, 1e-6,
                           False, 48, 16, 32),
    # Qwen3-0.6B shape, contiguous KV; 512 prompt tokens + 256 greedy tokens
    "qwen3-0.6b": ModelShape("qwen3-0.6b", 4, 28, 1024, 16, 8, 128, 3072, 151936, True,
                             True, 1e6, 128, 1e-6, False, 768, 512, 256),
    # two layers of the Qwen3-8B family's proportions that fit the persistent
    # layer kernel (hidden 2048, 16/4 heads of 128, SwiGLU 6144), paged KV;
    # 136 prompt tokens + 24 greedy tokens (two 128-key attention splits)
    "layerk": ModelShape("layerk", 6, 2, 2048, 16, 4, 128, 6144, 4096, False, True, 1e6, 128,
                         1e-6, True, 320, 136, 24),
    # Qwen3-8B shape, untied head, paged KV (block 16, shuffled table);
    # 2048 prompt tokens + 512 greedy tokens
    "qwen3-8b": ModelShape("qwen3-8b", 5, 36, 4096, 32, 8, 128, 12288, 151936, False,
                           True, 1e6, 128, 1e-6, True, 2560, 2048, 512),
}

# isolated q4_0 GEMV sweep (N rows, K cols): o-proj, fused qkv, fused gate|up,
# down, LM head of the Qwen3-8B shape
GEMV_SHAPES = [(4096, 4096), (6144, 4096), (24576, 4096), (4096, 12288), (151936, 4096)]
GEMV_SEED = 2

# isolated GQA decode attention
ATTN_SEED = 3
ATTN_NQ, ATTN_NKV, ATTN_HD, ATTN_BLOCK = 32, 8, 128, 16
ATTN_CASES = {
    "b1_kv512": (1, [512]),
    "b1_kv4096": (1, [4096]),
    "b1_kv32768": (1, [32768]),
    "b8_mixed": (8, None),   # kv_len ~ U{1..16384}, drawn from the seed
}
ATTN_B8_MAX = 16384


def _ss(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=key)))


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


# --------------------------------------------------------------------------- q4_0 packing

def quantize_q4_0(w: np.ndarray):
    """Pack an f32 matrix ``[rows, cols]`` into q4_0 (harness side only).

    Per 32-element block: ``m`` is the element of largest magnitude (signed,
    first one on ties), the scale is ``d = m / -8`` stored as binary16 (round to
    nearest even), and each code is ``clamp(rint(x / d) + 8, 0, 15)`` computed
    with the stored scale, so ``m`` itself maps exactly to code 0.  A block of
    zeros gets ``d = 0`` and codes 8.
    """
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, cols = w.shape
    if cols % 32:
        raise ValueError("q4_0 needs cols % 32 == 0")
    nb = cols // 32
    blk = w.reshape(rows, nb, 32)
    idx = np.abs(blk).argmax(axis=2)
    m = np.take_along_axis(blk, idx[..., None], axis=2)[..., 0]
    d16 = (m / np.float32(-8.0)).astype(np.float16)
    dq = d16.astype(np.float32)
    with np.errstate(divide="ignore"):
        inv = np.where(dq != 0, np.float32(1.0) / dq, np.float32(0.0)).astype(np.float32)
    q = np.rint(blk * inv[..., None]) + np.float32(8.0)
    q = np.clip(q, 0, 15).astype(np.uint8)
    qs = (q[..., :16] | (q[..., 16:] << 4)).astype(np.uint8)
    return np.ascontiguousarray(d16.view(np.uint16)), np.ascontiguousarray(qs)


@dataclass
class Q4Matrix:
    d: np.ndarray    # uint16 [rows, cols/32]
    qs: np.ndarray   # uint8 [rows, cols/32, 16]

    @property
    def rows(self) -> int:
        return self.d.shape[0]

    @property
    def cols(self) -> int:
        return self.d.shape[1] * 32

    @property
    def nbytes(self) -> int:
        return self.d.nbytes + self.qs.nbytes


def _q4_alloc(rows: int, cols: int) -> Q4Matrix:
    return Q4Matrix(np.empty((rows, cols // 32), dtype=np.uint16),
                    np.empty((rows, cols // 32, 16), dtype=np.uint8))


def _q4_chunks(m: Q4Matrix, seed: int, tensor_id: int):
    """Work items filling ``m`` from N(0, WEIGHT_STD) draws, one per row chunk."""
    rows, cols = m.rows, m.cols
    rchunk = max(1, ROW_CHUNK_ELEMS // cols)

    def work(ci: int):
        r0 = ci * rchunk
        r1 = min(rows, r0 + rchunk)
        g = _ss(seed, tensor_id, ci)
        w = g.standard_normal((r1 - r0, cols), dtype=np.float32) * np.float32(WEIGHT_STD)
        m.d[r0:r1], m.qs[r0:r1] = quantize_q4_0(w)

    return [(work, ci) for ci in range((rows + rchunk - 1) // rchunk)]


def _run(items, workers: int):
    if workers <= 1 or len(items) <= 1:
        for f, a in items:
            f(a)
        return
    with _cf.ThreadPoolExecutor(max_workers=workers) as pool:
        for _ in pool.map(lambda it: it[0](it[1]), items):
            pass


def random_q4_matrix(seed: int, tensor_id: int, rows: int, cols: int,
                     workers: int = 1) -> Q4Matrix:
    """q4_0 matrix from N(0, WEIGHT_STD) f32 draws, drawn in row chunks."""
    m = _q4_alloc(rows, cols)
    _run(_q4_chunks(m, seed, tensor_id), workers)
    return m


def random_norm(seed: int, tensor_id: int, n: int) -> np.ndarray:
    g = _ss(seed, tensor_id, 0)
    return (np.float32(1.0) + g.standard_normal(n, dtype=np.float32) * np.float32(NORM_STD)).astype(np.float32)


def rope_inv_freq(theta: float, rot_dim: int) -> np.ndarray:
    """inv_freq[i] = theta^(-2i/rot_dim) in f64, rounded to f32 (the host-precomputed input)."""
    i = np.arange(rot_dim // 2, dtype=np.float64)
    return (float(theta) ** (-(2.0 * i) / float(rot_dim))).astype(np.float32)


# --------------------------------------------------------------------------- models

@dataclass
class LayerWeights:
    wq: Q4Matrix
    wk: Q4Matrix
    wv: Q4Matrix
    wo: Q4Matrix
    wgate: Q4Matrix
    wup: Q4Matrix
    wdown: Q4Matrix
    attn_norm: np.ndarray
    ffn_norm: np.ndarray
    q_norm: np.ndarray
    k_norm: np.ndarray
    attn_gate: Q4Matrix | None = None   # attention output gate rows [n_heads*hd, H], if any


@dataclass
class ModelInputs:
    shape: ModelShape
    embed: Q4Matrix
    layers: list
    final_norm: np.ndarray
    lm_head: Q4Matrix          # same object as embed when tied
    inv_freq: np.ndarray
    prompt: np.ndarray         # int32 [prompt_len]
    block_table: np.ndarray    # int32 [ceil(max_seq/block)] (paged) or empty
    digest: str = field(default="")


# tensor ids: 0 embed, 1 final_norm, 2 lm_head, 3 prompt, 4 block table,
# 16 + 16*layer + k for the per-layer tensors
_T_EMBED, _T_FINAL, _T_LM, _T_PROMPT, _T_TABLE = 0, 1, 2, 3, 4


def _lt(layer: int, k: int) -> int:
    return 16 + 16 * layer + k


def make_model(name_or_shape, workers: int | None = None, attn_out_gate: bool = False) -> ModelInputs:
    """Seeded inputs of a model.  attn_out_gate adds an attention output gate
    matrix per layer, drawn from tensor ids of its own: every other tensor is
    the same as without it."""
    s = MODELS[name_or_shape] if isinstance(name_or_shape, str) else name_or_shape
    H, hd, I = s.hidden, s.head_dim, s.intermediate
    nq, nkv = s.n_heads * hd, s.n_kv * hd
    workers = workers or _workers()
    items = []

    def mat(tid, r, c):
        m = _q4_alloc(r, c)
        items.extend(_q4_chunks(m, s.seed, tid))
        return m

    embed = mat(_T_EMBED, s.vocab, H)
    layers = []
    for li in range(s.layers):
        shapes = [(nq, H), (nkv, H), (nkv, H), (H, nq), (I, H), (I, H), (H, I)]
        ms_ = [mat(_lt(li, k), r, c) for k, (r, c) in enumerate(shapes)]
        layers.append(LayerWeights(*ms_,
                                   attn_norm=random_norm(s.seed, _lt(li, 7), H),
                                   ffn_norm=random_norm(s.seed, _lt(li, 8), H),
                                   q_norm=random_norm(s.seed, _lt(li, 9), hd),
                                   k_norm=random_norm(s.seed, _lt(li, 10), hd),
                                   attn_gate=mat(_lt(li, 11), nq, H) if attn_out_gate else None))
    lm = embed if s.tied else mat(_T_LM, s.vocab, H)
    # largest chunks first keeps the pool busy to the end
    items.sort(key=lambda it: -it[1])
    _run(items, workers)
    final_norm = random_norm(s.seed, _T_FINAL, H)
    prompt = _ss(s.seed, _T_PROMPT, 0).integers(0, s.vocab, size=s.prompt_len, dtype=np.int64).astype(np.int32)
    if s.kv_paged:
        nblk = (s.max_seq + s.kv_block_size - 1) // s.kv_block_size
        if s.shuffle_blocks:
            table = _ss(s.seed, _T_TABLE, 0).permutation(nblk).astype(np.int32)
        else:
            table = np.arange(nblk, dtype=np.int32)
    else:
        table = np.zeros(0, dtype=np.int32)
    mi = ModelInputs(s, embed, layers, final_norm, lm, rope_inv_freq(s.rope_theta, s.rot_dim),
                     prompt, table)
    mi.digest = model_digest(mi)
    return mi


def model_digest(mi: ModelInputs) -> str:
    """SHA-256 over every input array of a model, in a fixed order."""
    h = hashlib.sha256()

    def add(a):
        h.update(np.ascontiguousarray(a).tobytes())

    add(mi.embed.d); add(mi.embed.qs)
    for L in mi.layers:
        for m in (L.wq, L.wk, L.wv, L.wo, L.wgate, L.wup, L.wdown):
            add(m.d); add(m.qs)
        for v in (L.attn_norm, L.ffn_norm, L.q_norm, L.k_norm):
            add(v)
        if L.attn_gate is not None:   # only when present: digests of ungated models unchanged
            add(L.attn_gate.d); add(L.attn_gate.qs)
    add(mi.final_norm)
    if not mi.shape.tied:
        add(mi.lm_head.d); add(mi.lm_head.qs)
    add(mi.inv_freq); add(mi.prompt); add(mi.block_table)
    return h.hexdigest()


# --------------------------------------------------------------------------- GEMV sweep

def gemv_case(shape_index: int, copies: int = 1):
    """(W copies, x) for sweep shape ``GEMV_SHAPES[shape_index]``; x ~ N(0,1) f32.

    Copy ``c`` of the matrix is drawn from its own seed, so rotating through the
    copies streams distinct bytes."""
    N, K = GEMV_SHAPES[shape_index]
    mats = [random_q4_matrix(GEMV_SEED, 100 * shape_index + c, N, K, _workers()) for c in range(copies)]
    x = _ss(GEMV_SEED, 100 * shape_index + 99, 0).standard_normal(K, dtype=np.float32)
    return mats, x


def random_gemv(seed: int, N: int, K: int, x_scale: float = 1.0):
    """Small GEMV case of any shape (K % 32 == 0)."""
    W = random_q4_matrix(seed, 1, N, K)
    x = (_ss(seed, 2, 0).standard_normal(K, dtype=np.float32) * np.float32(x_scale)).astype(np.float32)
    return W, x


def random_experts(seed: int, n_experts: int, N: int, K: int) -> Q4Matrix:
    """A stack of n_experts q4_0 matrices [N, K] (weights N(0, 0.02)) as one
    [n_experts * N, K] matrix: expert e is rows e*N .. (e+1)*N."""
    return random_q4_matrix(seed, 5, n_experts * N, K, _workers())


def expert_rows(W: Q4Matrix, e: int, N: int) -> Q4Matrix:
    """Expert e of a stack as its own matrix (a view)."""
    return Q4Matrix(W.d[e * N:(e + 1) * N], W.qs[e * N:(e + 1) * N])


def batch_x(seed: int, B: int, K: int) -> np.ndarray:
    """B input vectors of a batched GEMV case: f32 [B, K], N(0,1), each row from
    its own seed key."""
    return np.stack([_ss(seed, 3, b).standard_normal(K, dtype=np.float32) for b in range(B)]) \
        if B > 0 else np.zeros((0, K), np.float32)


# --------------------------------------------------------------------------- fp8 e4m3 (harness)

def _e4m3_table() -> np.ndarray:
    """Values of the 256 OCP e4m3 codes (sign, 4-bit exponent with bias 7, 3-bit
    mantissa; exponent 0 subnormal; 0x7f / 0xff NaN, no infinities)."""
    c = np.arange(256)
    sgn = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    v = sgn * mag
    v[(c & 0x7F) == 0x7F] = np.nan
    return v


def quantize_e4m3(x: np.ndarray) -> np.ndarray:
    """f32/f64 -> e4m3 code bytes, round to nearest (ties to the even code),
    saturating at +-448 (input generation for the fp8 KV cases; NaN refused)."""
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any():
        raise ValueError("NaN has no finite e4m3 code")
    pos = _e4m3_table()[:127]                      # codes 0 .. 126: 0 .. 448, increasing
    a = np.minimum(np.abs(x), 448.0)
    hi = np.clip(np.searchsorted(pos, a, side="left"), 0, 126)
    lo = np.maximum(hi - 1, 0)
    dl, dh = a - pos[lo], pos[hi] - a
    pick_hi = (dh < dl) | ((dh == dl) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)   # -0 keeps its sign


# --------------------------------------------------------------------------- attention

@dataclass
class AttnInputs:
    q: np.ndarray             # f32 [B, nq, hd]
    k_pool: np.ndarray        # uint16 (f16 bits) [num_blocks, nkv, block, hd]
    v_pool: np.ndarray        # same
    block_tables: np.ndarray  # int32 [B, max_blocks_per_seq] (-1 past a sequence's end)
    kv_lens: np.ndarray       # int32 [B]
    nq: int
    nkv: int
    hd: int
    block: int

    @property
    def B(self):
        return self.q.shape[0]

    @property
    def max_kv_len(self):
        return int(self.kv_lens.max()) if len(self.kv_lens) else 0


def random_attn(seed: int, B: int, kv_lens, nq=ATTN_NQ, nkv=ATTN_NKV, hd=ATTN_HD,
                block=ATTN_BLOCK, spare_blocks: int = 3, shuffle: bool = True) -> AttnInputs:
    """Paged decode-attention inputs: q ~ N(0,1) f32; K, V ~ N(0,1) rounded to f16;
    a pool of sum(ceil(kv_len/block)) + spare blocks; each sequence's logical
    blocks map to physical blocks through a seeded random permutation."""
    kv_lens = np.asarray(kv_lens, dtype=np.int32)
    assert kv_lens.shape == (B,)
    nblk_seq = (kv_lens + block - 1) // block
    total = int(nblk_seq.sum()) + spare_blocks
    perm = _ss(seed, 10, 0).permutation(total).astype(np.int32) if shuffle \
        else np.arange(total, dtype=np.int32)
    mbps = max(1, int(nblk_seq.max()) if B else 1)
    tables = np.full((B, mbps), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        n = int(nblk_seq[b])
        tables[b, :n] = perm[off:off + n]
        off += n
    q = _ss(seed, 11, 0).standard_normal((B, nq, hd), dtype=np.float32)
    pool_shape = (total, nkv, block, hd)
    k = np.empty(pool_shape, dtype=np.float16)
    v = np.empty(pool_shape, dtype=np.float16)
    per = max(1, (1 << 22) // (nkv * block * hd))

    def fill(arr, tid):
        for ci, b0 in enumerate(range(0, total, per)):
            b1 = min(total, b0 + per)
            arr[b0:b1] = _ss(seed, tid, ci).standard_normal((b1 - b0,) + pool_shape[1:],
                                                            dtype=np.float32)
    with _cf.ThreadPoolExecutor(max_workers=2) as pool:
        list(pool.map(lambda a: fill(*a), [(k, 12), (v, 13)]))
    return AttnInputs(q, k.view(np.uint16), v.view(np.uint16), tables, kv_lens,
                      nq, nkv, hd, block)


def attn_case(name: str) -> AttnInputs:
    B, lens = ATTN_CASES[name]
    if lens is None:
        lens = _ss(ATTN_SEED, 20, 0).integers(1, ATTN_B8_MAX + 1, size=B).astype(np.int32)
    return random_attn(ATTN_SEED, B, lens)


def contiguous_from_paged(a: AttnInputs, max_kv: int | None = None):
    """The same K/V laid out contiguously ``[B, nkv, max_kv, hd]`` (uint16 f16 bits),
    gathered through the block tables; slots past kv_len are zero."""
    max_kv = max_kv or max(1, a.max_kv_len)
    kc = np.zeros((a.B, a.nkv, max_kv, a.hd), dtype=np.uint16)
    vc = np.zeros_like(kc)
    for b in range(a.B):
        n = int(a.kv_lens[b])
        for lb in range((n + a.block - 1) // a.block):
            t0 = lb * a.block
            t1 = min(n, t0 + a.block)
            p = int(a.block_tables[b, lb])
            kc[b, :, t0:t1] = a.k_pool[p, :, : t1 - t0]
            vc[b, :, t0:t1] = a.v_pool[p, :, : t1 - t0]
    return kc, vc
