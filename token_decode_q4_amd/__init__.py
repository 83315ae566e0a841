"""MI355X (gfx950) batch-1 q4_0 decode: a C-ABI HIP library and its binding.

The library (``libqd.so``, C ABI in ``include/qd.h``) holds the whole decode
path: q4_0 GEMV, split-KV GQA decode attention, fused norm / rotary / SwiGLU /
residual epilogues and the hipGraph-replayed step.  ``_native`` is the thin
ctypes binding used by the tests and the benchmark.
"""
from ._native import (EXPORTS, LIB_PATH, Model, QdError, attn_decode,  # noqa: F401
                      attn_decode_kv8, attn_decode_noalloc, attn_noalloc_max_bytes,
                      attn_workspace_bytes, check, gemv_q4_0, gemv_q4_0_batch,
                      gemv_q4_0_experts, lib, prefill_chunk,
                      rope_inv_freq, stream_read,
                      stream_read_groups)
