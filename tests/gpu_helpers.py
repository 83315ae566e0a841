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



# lines repeated in the session's terminal summary (compared greedy counts and
# logit errors), so they show even when passing tests' output is captured
SUMMARY: list = []


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


def record(line: str):
    say(line)
    SUMMARY.append(line)


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


def check_greedy(gpu_tokens, ref_tokens, ref_margins, label: str, step_err=None):
    """Greedy tokens must be equal.  A first difference at step i is accepted
    only as a near-tie: the oracle's top-1 minus top-2 margin at i must be below
    the logit error measured at that same step, step_err(i) (max |gpu - oracle|
    over the step's compared logits; None when that step's logits are not
    available, and then nothing is accepted).  The sequences are not comparable
    after an accepted tie.  Returns (number of equal leading tokens, whether a
    tie was accepted); the count is printed."""
    G = len(ref_tokens)
    i = first_mismatch(gpu_tokens, ref_tokens)
    if i >= G:
        record(f"{label}: {G}/{G} greedy tokens equal (min oracle margin {float(np.min(ref_margins)):.3e})")
        return G, False
    m = float(ref_margins[i])
    e = step_err(i) if step_err is not None else None
    record(f"{label}: {i}/{G} greedy tokens equal; step {i}: gpu {int(gpu_tokens[i])} vs oracle "
        f"{int(ref_tokens[i])}, oracle top-2 margin {m:.3e}, measured logit error at that step "
        f"{'not available' if e is None else f'{e:.3e}'}")
    assert e is not None and m < e, f"{label}: greedy token {i} differs (margin {m:.3e}, error {e})"
    record(f"{label}: step {i} accepted as a near-tie (margin below the measured error)")
    return i, True
