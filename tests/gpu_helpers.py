"""Shared helpers of the GPU parity tests (device tensors, error measures,
greedy comparison).  Imported by the ``-m gpu`` tests only."""
from __future__ import annotations

import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden")

# Bars (the benchmark spec): GEMV outputs max relative error <= 1e-3 (normwise,
# max |y - y_ref| / max |y_ref|), final logits max abs error <= 2e-2.
GEMV_BAR = 1e-3
LOGITS_BAR = 2e-2
# Greedy near-tie: a differing token counts as a tie only when the oracle's
# top-1 minus top-2 logit margin is below this (well above the f32-vs-f64
# logit error measured on these configs, far below the typical margin).
TIE_MARGIN = 1e-3


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


def dev(a, dtype=None):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    t = torch.from_numpy(a)
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def host(t) -> np.ndarray:
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def normwise(y, ref) -> float:
    m = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(np.asarray(y, np.float64) - ref))) / (m if m > 0 else 1.0)


def load_golden(name: str):
    p = os.path.join(GOLDEN, f"greedy_{name}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        return json.load(f)


def first_mismatch(a, b) -> int:
    n = min(len(a), len(b))
    for i in range(n):
        if int(a[i]) != int(b[i]):
            return i
    return n if len(a) == len(b) else n


def check_greedy(gpu_tokens, ref_tokens, ref_margins, label: str) -> int:
    """Greedy tokens must be equal.  A first difference is accepted only as a
    near-tie (oracle margin < TIE_MARGIN); the sequences are not comparable
    after it.  Returns the number of compared (equal) tokens."""
    i = first_mismatch(gpu_tokens, ref_tokens)
    if i < len(ref_tokens):
        m = float(ref_margins[i])
        say(f"{label}: first greedy difference at step {i}: gpu {int(gpu_tokens[i])} vs oracle "
            f"{int(ref_tokens[i])}, oracle top-2 margin {m:.3e}")
        assert m < TIE_MARGIN, f"{label}: greedy token {i} differs with margin {m:.3e}"
    else:
        say(f"{label}: all {len(ref_tokens)} greedy tokens equal "
            f"(min oracle margin {float(np.min(ref_margins)):.3e})")
    return i
