"""Write the oracle's expected greedy decode for a model config.

Calls only ``oracle`` and ``synth``.  For the config named on the command
line it prefills the seeded prompt by sequential decode, generates the greedy
tokens, and stores, as JSON next to this script:

* the SHA-256 of every input array (so a mismatch of inputs is detected);
* the greedy tokens and the oracle's top-1 minus top-2 logit margin at each
  greedy step;
* sampled logits at a few steps: 2048 seeded vocab indices plus the oracle's
  top 16 at prefill positions 0 and P/2 and at greedy steps 0, 1, G/2 and G-1.

Usage: python tests/golden/make_golden.py qwen3-0.6b [--threads N]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth   # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))
N_SAMPLE = 2048


def sample_indices(vocab: int, seed: int) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(777,))))
    return np.sort(g.choice(vocab, size=min(N_SAMPLE, vocab), replace=False)).astype(np.int64)


def golden_path(name: str) -> str:
    return os.path.join(HERE, f"greedy_{name}.json")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("config", choices=sorted(synth.MODELS))
    ap.add_argument("--threads", type=int, default=None)
    args = ap.parse_args()
    t0 = time.time()
    mi = synth.make_model(args.config)
    s = mi.shape
    print(f"[golden] {s.name}: inputs ready in {time.time() - t0:.1f}s digest {mi.digest}", flush=True)
    model = oracle.Model(mi, nthreads=args.threads)
    P, G = s.prompt_len, s.gen
    idx = sample_indices(s.vocab, s.seed)
    prefill_at = sorted({0, P // 2})
    greedy_at = sorted({0, 1, G // 2, G - 1})
    samples = {}

    def keep(tag, lg):
        top = np.argsort(-lg, kind="stable")[:16]
        samples[tag] = {"idx": idx.tolist(), "val": [float(v) for v in lg[idx]],
                        "top_idx": top.tolist(), "top_val": [float(v) for v in lg[top]]}

    toks, margins = [], []
    cur = int(mi.prompt[0])
    t1 = time.time()
    for pos in range(P + G - 1):
        lg = model.step(cur, pos)
        if pos < P - 1:
            if pos in prefill_at:
                keep(f"prefill:{pos}", lg)
            cur = int(mi.prompt[pos + 1])
        else:
            gi = pos - (P - 1)
            t, m = oracle.greedy_pick(lg)
            toks.append(t)
            margins.append(m)
            if gi in greedy_at:
                keep(f"greedy:{gi}", lg)
            cur = t
        if pos % 64 == 0:
            el = time.time() - t1
            print(f"[golden] pos {pos}/{P + G - 1} {el:.0f}s ({el / (pos + 1):.3f}s/step)", flush=True)
    out = {
        "config": s.name,
        "digest": mi.digest,
        "prompt_len": P,
        "gen": G,
        "tokens": [int(t) for t in toks],
        "margins": [float(m) for m in margins],
        "samples": samples,
        "oracle_threads": model.nthreads,
        "oracle_seconds": time.time() - t1,
        "written_by": "python tests/golden/make_golden.py " + s.name,
    }
    with open(golden_path(s.name) + ".tmp", "w") as f:
        json.dump(out, f)
    os.replace(golden_path(s.name) + ".tmp", golden_path(s.name))
    print(f"[golden] wrote {golden_path(s.name)} in {time.time() - t0:.0f}s", flush=True)


if __name__ == "__main__":
    main()
