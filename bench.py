"""Benchmark: batch-1 greedy decode tok/s at the Qwen3-8B shape on one MI355X.

One timed "step" is one decode step of the whole path (embedding, 36 layers of
fused q4_0 GEMVs + split-KV GQA attention + fused norm/rotary/SwiGLU/residual,
LM head + greedy argmax), replayed from a hipGraph with the token and position
held on the device.  The 2048-token seeded prompt is prefilled by sequential
decode first; warmup and timed steps are the greedy steps that follow
(positions 2047 + ...), as in the 2048 + 512 workload.

Also reported, on the same JSON line:
  roofline      the q4_0 GEMV at the fused gate|up shape (24576 x 4096, the
                step's largest kernel) through qd_gemv_q4_0 -- the same kernel
                template and launch configuration as the step's gate|up GEMV --
                100 launches over >= 1 GiB of rotated weight copies (no launch
                hits the Infinity Cache) captured in one graph and timed with
                HIP events on the replay stream; achieved = algorithmic bytes /
                mean launch duration, against 8 TB/s.  traffic = HBM bytes per
                launch from the committed rocprofv3 PMC record
                (profiles/gemv_q4_0_24576x4096_traffic.md) while the kernel
                sources still match it, else null.
  step_roofline the whole step's algorithmic bytes / measured step time.
  cpu_baseline  the f64 CPU oracle running decode steps of the same model on
                the host cores, a bounded sample at the first positions the
                GPU timed (same kv_len; the CPU model and thread count named).

  rows          per-row measurements: the isolated GEMV at the five sweep
                shapes, the batched and the expert GEMV, and the isolated
                attention at the four cases (f16 and fp8 caches) (graphs of
                100 launches over >= 1 GiB of rotated copies, each output
                checked against the f64 oracle, the oracle's host time beside
                it), greedy decode at the Qwen3-0.6B shape, and batched decode
                of 4, 8 and 16 sequences at the benchmarked shape.

Usage: python bench.py [--gpus 1] [--steps 448] [--warmup 16] [--no-rows]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def q4_bytes(rows: int, cols: int) -> int:
    return rows * cols * 18 // 32


def step_bytes(s, kv_len: int, kv_bytes: int = 2) -> int:
    """Algorithmic HBM bytes of one decode step at context kv_len (K/V read for
    kv_len positions, one position written): q4_0 weights (+ the embedding row),
    f32 norm vectors, the K/V traffic at kv_bytes per element (2 for the f16
    cache, 1 for fp8)."""
    H, I, hd, nq, nkv, V, L = s.hidden, s.intermediate, s.head_dim, s.n_heads, s.n_kv, s.vocab, s.layers
    per_layer = (q4_bytes((nq + 2 * nkv) * hd, H) + q4_bytes(H, nq * hd) + q4_bytes(2 * I, H)
                 + q4_bytes(H, I) + 4 * (2 * H + 2 * hd))
    kv = L * (kv_len * nkv * hd * kv_bytes * 2 + nkv * hd * kv_bytes * 2)
    return L * per_layer + q4_bytes(V, H) + q4_bytes(1, H) + 4 * H + kv


GEMV_SHAPE = (24576, 4096)   # the gate|up GEMV of the step, the largest per-layer kernel
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "gemv_q4_0_24576x4096_traffic.md")
KERNEL_SOURCES = ["gemv_q4_0.h", "qd_common.h", "gemv_cfg.h"]   # kernel + its launch configuration


def kernel_source_digest() -> str:
    """SHA-256 over the sources that define the timed GEMV kernel and its launch."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "token_decode_q4_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def stored_traffic():
    """HBM bytes per launch from the committed PMC record, if it was taken on the
    kernel as it is now (same source digest); else None."""
    try:
        with open(TRAFFIC_RECORD) as fh:
            for line in fh:
                if line.startswith("traffic_record:"):
                    rec = json.loads(line.split(":", 1)[1])
                    if rec.get("kernel_src_sha256") == kernel_source_digest():
                        return rec
    except OSError:
        pass
    return None


def gemv_roofline(reps: int = 100, min_bytes: int = 1 << 30):
    """qd_gemv_q4_0 at 24576 x 4096 (config 2's gate|up shape, the same kernel
    template and launch configuration as the step's gate|up GEMV): `reps`
    launches over rotated weight copies (>= 1 GiB, so no launch hits the
    Infinity Cache), captured in one graph and replayed; HIP events on the
    replay stream give the mean launch duration.  Also runs one 1 GiB
    device-to-device copy, the known-size reference for the PMC byte
    counters."""
    import torch
    import synth
    import token_decode_q4_amd as qd
    N, K = GEMV_SHAPE
    (W,), x = synth.gemv_case(synth.GEMV_SHAPES.index((N, K)))
    nbytes_w = W.d.nbytes + W.qs.nbytes
    copies = max(1, -(-min_bytes // nbytes_w))
    d0 = torch.from_numpy(W.d.view(np.int16)).cuda()
    q0 = torch.from_numpy(W.qs).cuda()
    ds = [d0] + [d0.clone() for _ in range(copies - 1)]
    qs = [q0] + [q0.clone() for _ in range(copies - 1)]
    xt = torch.from_numpy(x).cuda()
    y = torch.empty(N, dtype=torch.float32, device="cuda")
    stream = torch.cuda.Stream()
    us = _graph_time(stream, lambda i: qd.gemv_q4_0(ds[i % copies], qs[i % copies], xt, y,
                                                    stream=stream), reps)
    with torch.cuda.stream(stream):
        # the known-size copy for the byte counters
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        stream.synchronize()
        del src, dst
    algo = N * K * 18 // 32 + 4 * K + 4 * N
    achieved = algo / (us * 1e-6) / 1e9
    rec = stored_traffic()
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": rec["bytes_per_launch"] if rec else None,
            "kernel": f"k_gemv_plain (qd_gemv_q4_0) {N}x{K}, graph of {reps} launches "
                      f"replayed {TIMED_REPLAYS} times",
            "mean_us": round(us, 3), "bytes_per_launch": algo, "weight_copies": copies}


TIMED_REPLAYS = 10


def _graph_time(stream, launch, reps: int, replays: int = TIMED_REPLAYS) -> float:
    """Mean microseconds per launch: 10 warm-up launches, then `reps` launches
    captured in one graph, replayed once untimed and then `replays` times back
    to back between two HIP events on the replay stream (the mean over
    reps x replays launches)."""
    import torch
    with torch.cuda.stream(stream):
        for i in range(10):
            launch(i)
        stream.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for i in range(reps):
                launch(i)
        graph.replay()
        stream.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(replays):
            graph.replay()
        e1.record(stream)
        stream.synchronize()
        del graph
    return e0.elapsed_time(e1) * 1e3 / (reps * replays)


def _timed(fn, reps: int = 3):
    """(best wall seconds of `reps` calls, the last result)"""
    best, r = float("inf"), None
    for _ in range(reps):
        t0 = time.perf_counter()
        r = fn()
        best = min(best, time.perf_counter() - t0)
    return best, r


def gemv_sweep_rows(reps: int = 100, min_bytes: int = 1 << 30):
    """The isolated q4_0 GEMV at the five sweep shapes through qd_gemv_q4_0:
    `reps` launches over >= 1 GiB of rotated weight copies in one graph (no
    launch hits the Infinity Cache); the output of the first launch against
    the f64 oracle (normwise error); the oracle's own time on the host cores
    (best of 3), as GB/s of the same algorithmic bytes."""
    import torch
    import oracle
    import synth
    import token_decode_q4_amd as qd
    rows, tot_bytes, tot_us = [], 0, 0.0
    for i, (N, K) in enumerate(synth.GEMV_SHAPES):
        (W,), x = synth.gemv_case(i)
        copies = max(1, -(-min_bytes // (W.d.nbytes + W.qs.nbytes)))
        d0 = torch.from_numpy(W.d.view(np.int16)).cuda()
        q0 = torch.from_numpy(W.qs).cuda()
        ds = [d0] + [d0.clone() for _ in range(copies - 1)]
        qs = [q0] + [q0.clone() for _ in range(copies - 1)]
        xt = torch.from_numpy(x).cuda()
        y = torch.empty(N, dtype=torch.float32, device="cuda")
        stream = torch.cuda.Stream()
        with torch.cuda.stream(stream):
            qd.gemv_q4_0(d0, q0, xt, y, stream=stream)
        stream.synchronize()
        got = y.cpu().numpy().astype(np.float64)
        t_or, ref = _timed(lambda: oracle.gemv(W, x))
        err = float(np.max(np.abs(got - ref)) / max(1e-300, float(np.max(np.abs(ref)))))
        us = _graph_time(stream, lambda k: qd.gemv_q4_0(ds[k % copies], qs[k % copies], xt, y,
                                                        stream=stream), reps)
        algo = N * K * 18 // 32 + 4 * K + 4 * N
        gbs = algo / (us * 1e-6) / 1e9
        rows.append({"shape": f"{N}x{K}", "mean_us": round(us, 3), "achieved": round(gbs, 1),
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_launch": algo,
                     "weight_copies": copies, "normwise_err_vs_oracle": err,
                     "oracle_s": round(t_or, 4), "oracle_gbs": round(algo / t_or / 1e9, 2)})
        tot_bytes += algo
        tot_us += us
        del ds, qs, d0, q0, xt, y
        torch.cuda.empty_cache()
    agg = tot_bytes / (tot_us * 1e-6) / 1e9
    return rows, {"achieved": round(agg, 1), "frac": round(agg / HBM_PEAK_GBS, 4), "unit": "GB/s",
                  "note": "byte-weighted over the five shapes: total bytes / total mean launch time"}


def gemv_batch_rows(batches=(1, 2, 4, 8, 16), reps: int = 100, min_bytes: int = 1 << 30):
    """The batched GEMV (qd_gemv_q4_0_batch) at the gate|up shape 24576 x 4096:
    Y[b] = W X[b] for B vectors, every weight read once; `reps` launches over
    >= 1 GiB of rotated weight copies in one graph.  Algorithmic bytes =
    N*K*18/32 + 4*B*(K + N); vectors per second = B / mean launch time."""
    import torch
    import oracle
    import synth
    import token_decode_q4_amd as qd
    idx = synth.GEMV_SHAPES.index(GEMV_SHAPE)
    N, K = GEMV_SHAPE
    (W,), _ = synth.gemv_case(idx)
    copies = max(1, -(-min_bytes // (W.d.nbytes + W.qs.nbytes)))
    d0 = torch.from_numpy(W.d.view(np.int16)).cuda()
    q0 = torch.from_numpy(W.qs).cuda()
    ds = [d0] + [d0.clone() for _ in range(copies - 1)]
    qs = [q0] + [q0.clone() for _ in range(copies - 1)]
    rows = []
    for B in batches:
        X = synth.batch_x(9000 + B, B, K)
        xt = torch.from_numpy(X).cuda()
        Y = torch.empty((B, N), dtype=torch.float32, device="cuda")
        stream = torch.cuda.Stream()
        with torch.cuda.stream(stream):
            qd.gemv_q4_0_batch(d0, q0, xt, Y, stream=stream)
        stream.synchronize()
        got = Y.cpu().numpy().astype(np.float64)
        err = 0.0
        for b in range(B):
            ref = oracle.gemv(W, X[b])
            err = max(err, float(np.max(np.abs(got[b] - ref)) / float(np.max(np.abs(ref)))))
        us = _graph_time(stream, lambda i: qd.gemv_q4_0_batch(ds[i % copies], qs[i % copies], xt, Y,
                                                              stream=stream), reps)
        algo = N * K * 18 // 32 + 4 * B * (K + N)
        gbs = algo / (us * 1e-6) / 1e9
        rows.append({"shape": f"{N}x{K}", "batch": B, "mean_us": round(us, 3), "achieved": round(gbs, 1),
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_launch": algo,
                     "vectors_per_s": round(B / (us * 1e-6), 1), "normwise_err_vs_oracle": err})
        del xt, Y
    del ds, qs, d0, q0
    torch.cuda.empty_cache()
    return rows


def experts_row(reps: int = 100, min_bytes: int = 1 << 30):
    """The expert GEMV (qd_gemv_q4_0_experts) at a mixture-of-experts decode
    shape: 8 of 64 experts of 1536 x 2048 (gate|up of a 768-wide expert over a
    2048 hidden), stacks rotated over >= 1 GiB so every launch reads its
    experts cold.  Algorithmic bytes = 8 * (N*K*18/32 + 4N) + 4K."""
    import torch
    import oracle
    import synth
    import token_decode_q4_amd as qd
    E, N, K, k = 64, 1536, 2048, 8
    W = synth.random_experts(4242, E, N, K)
    x = synth.batch_x(4243, 1, K)[0]
    picks = np.array([2, 9, 17, 30, 33, 41, 50, 63], dtype=np.int32)
    stack = W.d.nbytes + W.qs.nbytes
    copies = max(1, -(-min_bytes // stack))
    d0 = torch.from_numpy(W.d.view(np.int16).reshape(E, N, -1)).cuda()
    q0 = torch.from_numpy(W.qs.reshape(E, N, K // 32, 16)).cuda()
    ds = [d0] + [d0.clone() for _ in range(copies - 1)]
    qs = [q0] + [q0.clone() for _ in range(copies - 1)]
    e_t = torch.from_numpy(picks).cuda()
    xt = torch.from_numpy(x).cuda()
    y = torch.empty((k, N), dtype=torch.float32, device="cuda")
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        qd.gemv_q4_0_experts(d0, q0, e_t, xt, y, stream=stream)
    stream.synchronize()
    got = y.cpu().numpy().astype(np.float64)
    err = 0.0
    for j, e in enumerate(picks):
        ref = oracle.gemv(synth.expert_rows(W, int(e), N), x)
        err = max(err, float(np.max(np.abs(got[j] - ref)) / float(np.max(np.abs(ref)))))
    us = _graph_time(stream, lambda i: qd.gemv_q4_0_experts(ds[i % copies], qs[i % copies], e_t, xt, y,
                                                            stream=stream), reps)
    algo = k * (N * K * 18 // 32 + 4 * N) + 4 * K
    gbs = algo / (us * 1e-6) / 1e9
    del ds, qs, d0, q0
    torch.cuda.empty_cache()
    return {"shape": f"{k} of {E} experts, {N}x{K}", "mean_us": round(us, 3), "achieved": round(gbs, 1),
            "frac": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_launch": algo, "stack_copies": copies,
            "normwise_err_vs_oracle": err}


def attention_rows(reps: int = 100, min_bytes: int = 1 << 30, kv8: bool = False):
    """The isolated GQA decode attention (qd_attn_decode: split + combine) at
    the four cases (32 q / 8 kv heads, head_dim 128, paged block 16, shuffled
    tables): `reps` launches over >= 1 GiB of rotated K/V pool replicas in one
    graph; the output against the f64 oracle (normwise error) and the oracle's
    time on the host cores.  Algorithmic bytes = K/V rows read (sum of kv_len x
    nkv x hd x 2 B x 2) + q and out (f32) + the block-table entries used.
    kv8: the same cases over an fp8 e4m3 cache (qd_attn_decode_kv8; the f16
    values through the harness quantizer, K/V scales 0.625 / 1.75): 1 byte
    per K/V element."""
    import torch
    import oracle
    import synth
    import token_decode_q4_amd as qd
    out_rows = []
    for name in sorted(synth.ATTN_CASES):
        a = synth.attn_case(name)
        max_kv = max(1, a.max_kv_len)
        ksc, vsc = 0.625, 1.75
        if kv8:
            k8 = synth.quantize_e4m3(a.k_pool.view(np.float16).astype(np.float64))
            v8 = synth.quantize_e4m3(a.v_pool.view(np.float16).astype(np.float64))
            pool_bytes = k8.nbytes + v8.nbytes
        else:
            pool_bytes = a.k_pool.nbytes + a.v_pool.nbytes
        copies = max(1, -(-min_bytes // pool_bytes))
        k0 = torch.from_numpy(k8 if kv8 else a.k_pool.view(np.int16)).cuda()
        v0 = torch.from_numpy(v8 if kv8 else a.v_pool.view(np.int16)).cuda()
        ks = [k0] + [k0.clone() for _ in range(copies - 1)]
        vs = [v0] + [v0.clone() for _ in range(copies - 1)]
        q = torch.from_numpy(np.ascontiguousarray(a.q)).cuda()
        lens = torch.from_numpy(np.ascontiguousarray(a.kv_lens)).cuda()
        tables = torch.from_numpy(np.ascontiguousarray(a.block_tables)).cuda()
        out = torch.empty((a.B, a.nq, a.hd), dtype=torch.float32, device="cuda")
        ws = torch.empty(qd.attn_workspace_bytes(a.B, a.nq, a.nkv, a.hd, max_kv), dtype=torch.uint8,
                         device="cuda")
        scale = 1.0 / np.sqrt(a.hd)
        stream = torch.cuda.Stream()

        def launch(k):
            if kv8:
                qd.attn_decode_kv8(q, ks[k % copies], vs[k % copies], lens, max_kv, a.nkv, scale, ksc,
                                   vsc, out, ws, block_tables=tables, stream=stream)
            else:
                qd.attn_decode(q, ks[k % copies], vs[k % copies], lens, max_kv, a.nkv, scale, out, ws,
                               block_tables=tables, stream=stream)

        with torch.cuda.stream(stream):
            launch(0)
        stream.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        if kv8:
            t_or, ref = _timed(lambda: oracle.attn_decode_e4m3(a.q, k8, v8, a.kv_lens, a.nkv, scale, ksc,
                                                               vsc, a.block_tables), reps=1)
        else:
            t_or, ref = _timed(lambda: oracle.attn_inputs(a), reps=1)
        err = float(np.max(np.abs(got - ref)) / max(1e-300, float(np.max(np.abs(ref)))))
        us = _graph_time(stream, launch, reps)
        kv = [int(v) for v in a.kv_lens]
        algo = (sum(kv) * a.nkv * a.hd * (1 if kv8 else 2) * 2 + 2 * a.B * a.nq * a.hd * 4
                + 4 * sum(-(-v // synth.ATTN_BLOCK) for v in kv))
        gbs = algo / (us * 1e-6) / 1e9
        out_rows.append({"case": name, "kv": "fp8 e4m3" if kv8 else "f16", "batch": a.B, "kv_lens": kv if a.B <= 8 else None,
                         "mean_us": round(us, 3), "achieved": round(gbs, 1),
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_launch": algo,
                         "pool_copies": copies, "normwise_err_vs_oracle": err,
                         "oracle_s": round(t_or, 4), "oracle_gbs": round(algo / t_or / 1e9, 2)})
        del ks, vs, k0, v0, q, lens, tables, out, ws
        torch.cuda.empty_cache()
    return out_rows


def decode_row(config: str, warmup: int = 16):
    """Greedy decode tok/s of another model shape through qd_generate (graph
    replays, no host sync): the prompt prefilled by sequential decode, then
    `warmup` untimed and the rest of the shape's greedy steps timed."""
    import torch
    import synth
    import token_decode_q4_amd as qd
    mi = synth.make_model(config)
    s = mi.shape
    P, G = s.prompt_len, s.gen
    model = qd.Model(mi, use_graph=True)
    toks = torch.empty(s.max_seq, dtype=torch.int32, device="cuda")
    model.set_prompt(mi.prompt)
    model.generate(0, P - 1 + warmup, tokens=toks[: P - 1 + warmup])
    torch.cuda.synchronize()
    pos, n = P - 1 + warmup, G - warmup
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    model.generate(pos, n, tokens=toks[pos:pos + n])
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    model.check()
    model.close()
    del model
    torch.cuda.empty_cache()
    mean_bytes = float(np.mean([step_bytes(s, k) for k in range(pos + 1, pos + n + 1)]))
    gbs = mean_bytes / (ms * 1e-3 / n) / 1e9
    return {"workload": f"{s.name} batch-1 greedy decode, positions {pos}..{pos + n - 1} after a "
                        f"{P}-token sequential-decode prefill", "steps": n,
            "tok_s": round(n / (ms * 1e-3), 1), "ms_per_step": round(ms / n, 4),
            "step_roofline": {"achieved": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
                              "unit": "GB/s", "bytes_per_step": round(mean_bytes)}}


def batch_decode_rows(mi, batches=(4, 8, 16), prompt: int = 512, warmup: int = 8, steps: int = 64):
    """Batched greedy decode at the model's shape (qd_create_batch): B
    sequences with their own seeded prompts of `prompt` tokens, prefilled by
    sequential batched steps, then `warmup` untimed and `steps` timed batched
    steps (graph replays, no host sync).  Aggregate tok/s = B * steps / time;
    paged K/V with a shuffled table per sequence."""
    import torch
    import token_decode_q4_amd as qd
    s = mi.shape
    out = []
    max_seq = prompt + warmup + steps
    need = (max_seq + 15) // 16
    for B in batches:
        rng = np.random.default_rng(1000 + B)
        table = rng.permutation(B * need).astype(np.int32).reshape(B, need)
        m = qd.Model(mi, batch=B, paged=True, max_seq=max_seq, block_table=table, num_kv_blocks=B * need)
        for b in range(B):
            m.set_prompt_seq(b, rng.integers(0, s.vocab, size=prompt).astype(np.int32))
        m.generate_batch([0] * B, prompt - 1 + warmup)
        torch.cuda.synchronize()
        pos = prompt - 1 + warmup
        stream = torch.cuda.current_stream()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        m.generate_batch([pos] * B, steps)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        m.check()
        m.close()
        del m
        torch.cuda.empty_cache()
        # bytes of a batched step: the weights once, each sequence's K/V (its
        # reads at its kv_len and its one written position)
        kv_w = s.layers * s.n_kv * s.head_dim * 2 * 2
        kv_seq = float(np.mean([step_bytes(s, k) - step_bytes(s, 0) for k in range(pos + 1, pos + steps + 1)])) + kv_w
        step_b = step_bytes(s, 0) - kv_w + B * kv_seq
        gbs = step_b / (ms * 1e-3 / steps) / 1e9
        out.append({"batch": B, "workload": f"{s.name} {B} sequences, {prompt}-token prompts, positions "
                                            f"{pos}..{pos + steps - 1}", "steps": steps,
                    "ms_per_step": round(ms / steps, 4), "tok_s": round(B * steps / (ms * 1e-3), 1),
                    "step_bytes": round(step_b), "achieved_gbs": round(gbs, 1),
                    "frac": round(gbs / HBM_PEAK_GBS, 4)})
        log(f"batched decode B={B}: {out[-1]['ms_per_step']} ms/step, {out[-1]['tok_s']} tok/s aggregate, "
            f"{gbs:.0f} GB/s")
    return out


def read_ceiling(nbytes: int, reps: int = 100, min_bytes: int = 1 << 30):
    """The measured ceiling the GEMV is compared with: qd_stream_read (plain
    128-bit non-temporal loads, nothing else) over `nbytes` per launch, the
    GEMV leg's launch pattern (`reps` launches over rotated slices of >= 1 GiB,
    one graph, HIP events on the replay stream); and one read of the whole
    >= 1 GiB buffer per launch."""
    import torch
    import token_decode_q4_amd as qd
    nbytes -= nbytes % 16
    copies = max(1, -(-min_bytes // nbytes))
    buf = torch.empty(copies * nbytes, dtype=torch.uint8, device="cuda")
    buf.random_(0, 256)
    sink = torch.empty(qd.stream_read_groups(copies * nbytes), dtype=torch.int32, device="cuda")
    stream = torch.cuda.Stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    us = _graph_time(stream, lambda i: qd.stream_read(buf[(i % copies) * nbytes:], sink, nbytes,
                                                      stream=stream), reps)
    with torch.cuda.stream(stream):
        big = copies * nbytes
        qd.stream_read(buf, sink, big, stream=stream)
        e0.record(stream)
        for _ in range(5):
            qd.stream_read(buf, sink, big, stream=stream)
        e1.record(stream)
        stream.synchronize()
        us_big = e0.elapsed_time(e1) * 1e3 / 5
    del buf, sink
    return {"kernel": f"k_stream_read (qd_stream_read), graph of {reps} launches replayed "
                      f"{TIMED_REPLAYS} times",
            "bytes_per_launch": nbytes, "mean_us": round(us, 3),
            "achieved": round(nbytes / (us * 1e-6) / 1e9, 1),
            "achieved_one_launch_of": big, "achieved_one_launch": round(big / (us_big * 1e-6) / 1e9, 1),
            "unit": "GB/s"}


def cpu_model_name() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(mi, pos0: int, tokens, seconds: float = 15.0):
    """The oracle as it stands, decode steps of the same model at the positions
    the GPU timed: positions pos0, pos0+1, ... fed `tokens` (the GPU's greedy
    tokens there), for about `seconds`.  The K/V of positions 0..pos0-1 are
    loaded with seeded f16 values instead of running those steps (the oracle
    needs minutes per hundred steps at this shape), so every timed step
    attends over the same kv_len as the GPU step at that position."""
    import oracle
    s = mi.shape
    threads = oracle.default_threads()
    om = oracle.Model(mi, nthreads=threads)
    kvd = s.n_kv * s.head_dim
    fill = np.random.default_rng(12345).standard_normal((pos0, kvd)).astype(np.float16).astype(np.float64)
    for layer in range(s.layers):
        om.load_kv(layer, 0, fill, fill)
    t0 = time.time()
    n = 0
    while True:
        om.step(int(tokens[n]), pos0 + n)
        n += 1
        if time.time() - t0 >= seconds or n >= len(tokens):
            break
    el = time.time() - t0
    om.close()
    return {"value": round(n / el, 4), "unit": "tok/s", "cores": threads, "kind": "oracle",
            "cpu": cpu_model_name(),
            "sample": f"{n} f64 oracle decode steps of the {s.name}-shape model at positions "
                      f"{pos0}..{pos0 + n - 1} (the first positions of the timed GPU steps, "
                      f"kv_len {pos0 + 1}..{pos0 + n}; K/V of positions 0..{pos0 - 1} loaded with "
                      f"seeded f16 values), {el:.1f} s on {threads} threads"}


def prefill_row(model, s, n: int, reps: int = 3):
    """Prompt positions 0..n-1 of a created model: chunked prefill (qd_prefill,
    chunks of qd_prefill_chunk() positions through the batched product) against prefill as sequential
    decode steps (qd_generate over the prompt).  The K/V cache is rewritten
    with the same values; each is timed with events around `reps` runs after
    one untimed run.  Weight bytes per chunk give its GB/s."""
    import torch
    import token_decode_q4_amd as qd
    stream = torch.cuda.current_stream()
    chunk = qd.prefill_chunk()

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    ms_c = timed(lambda: model.prefill(0, n))
    ms_s = timed(lambda: model.generate(0, n))
    model.check()
    chunks = -(-n // chunk)
    H, I = s.hidden, s.intermediate
    qkv = (s.n_heads + 2 * s.n_kv) * s.head_dim
    wbytes = s.layers * (q4_bytes(qkv, H) + q4_bytes(H, s.n_heads * s.head_dim) + q4_bytes(2 * I, H)
                         + q4_bytes(H, I))
    gbs = chunks * wbytes / (ms_c * 1e-3) / 1e9
    return {"workload": f"{s.name} prompt positions 0..{n - 1}", "positions": n, "chunk": chunk,
            "chunked_ms": round(ms_c, 3), "chunked_tok_s": round(n / (ms_c * 1e-3), 1),
            "sequential_ms": round(ms_s, 3), "sequential_tok_s": round(n / (ms_s * 1e-3), 1),
            "speedup": round(ms_s / ms_c, 2),
            "layer_weight_bytes_per_chunk": wbytes,
            "layer_weight_gbs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=448)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--config", default="qwen3-8b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-roofline", action="store_true")
    ap.add_argument("--kv-fp8", action="store_true",
                    help="fp8 e4m3 K/V cache (qd_config.kv_fp8; k_scale 0.5, v_scale 0.125)")
    ap.add_argument("--no-rows", action="store_true",
                    help="skip the per-row legs (GEMV sweep shapes, attention cases, 0.6B decode)")
    ap.add_argument("--layer-kernel", type=int, default=0,
                    help="1: one persistent kernel launch per layer (qd_config.layer_kernel)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="print only the prefill row (chunked vs sequential) of --config")
    ap.add_argument("--batch-only", action="store_true",
                    help="print only the batched decode rows of --config")
    ap.add_argument("--batch-sizes", default="4,8,16", help="sequences of the batched decode rows")
    ap.add_argument("--attention-only", action="store_true",
                    help="print only the standalone attention rows (f16 and fp8 caches)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): batch-1 decode of one "
              "model copy uses a single device.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import token_decode_q4_amd as qd

    torch.cuda.set_device(0)
    t0 = time.time()
    mi = synth.make_model(args.config)
    s = mi.shape
    log(f"inputs {s.name} ready in {time.time() - t0:.1f}s (sha256 {mi.digest[:16]})")
    P = s.prompt_len
    if P - 1 + args.warmup + args.steps > s.max_seq:
        sys.exit(f"warmup + steps must be <= {s.max_seq - P + 1}")
    if args.batch_only:
        print(json.dumps(batch_decode_rows(mi, tuple(int(b) for b in args.batch_sizes.split(",")))), flush=True)
        return
    if args.attention_only:
        a_rows = attention_rows() + attention_rows(kv8=True)
        for r in a_rows:
            log(f"attention {r['case']} {r['kv']}: {r['mean_us']} us, {r['achieved']} GB/s ({r['frac']:.3f})")
        print(json.dumps(a_rows), flush=True)
        return
    t0 = time.time()
    model = qd.Model(mi, use_graph=True, layer_kernel=bool(args.layer_kernel), kv_fp8=args.kv_fp8,
                     k_scale=0.5, v_scale=0.125)
    log(f"qd_create {time.time() - t0:.1f}s")
    if args.prefill_only:
        model.set_prompt(mi.prompt)
        print(json.dumps(prefill_row(model, s, P - 1)), flush=True)
        model.close()
        return
    stream = torch.cuda.current_stream()
    toks = torch.empty(s.max_seq, dtype=torch.int32, device="cuda")
    model.set_prompt(mi.prompt)
    t0 = time.time()
    model.generate(0, P - 1, tokens=toks[: P - 1])
    torch.cuda.synchronize()
    log(f"prefill {P - 1} steps in {time.time() - t0:.2f}s")
    pos = P - 1
    model.generate(pos, args.warmup, tokens=toks[pos:pos + args.warmup])
    pos += args.warmup
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    model.generate(pos, args.steps, tokens=toks[pos:pos + args.steps])
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    tok_s = args.steps / (ms * 1e-3)
    t_pos0 = pos
    toks_host = toks[pos - 1:pos - 1 + args.steps].cpu().numpy()   # the token fed at each position
    kv_lens = np.arange(pos + 1, pos + args.steps + 1)
    mean_bytes = float(np.mean([step_bytes(s, int(k), 1 if args.kv_fp8 else 2) for k in kv_lens]))
    step_gbs = mean_bytes / (ms * 1e-3 / args.steps) / 1e9
    log(f"decode {args.steps} steps: {ms:.2f} ms, {tok_s:.1f} tok/s, {step_gbs:.0f} GB/s")
    model.check()   # raises if the device recorded an error during the run
    pf_row = None if args.no_rows else prefill_row(model, s, P - 1)
    if pf_row:
        log(f"prefill {P - 1} positions: chunked {pf_row['chunked_tok_s']} tok/s, sequential decode "
            f"{pf_row['sequential_tok_s']} tok/s")
    model.close()
    del model
    torch.cuda.empty_cache()

    roof = None
    if not args.no_roofline:
        roof = gemv_roofline()
        log(f"gemv roofline: {roof['mean_us']} us, {roof['achieved']} GB/s")
        torch.cuda.empty_cache()
        ceil = read_ceiling(roof["bytes_per_launch"])
        roof["read_ceiling"] = ceil
        roof["frac_of_read_ceiling"] = round(roof["achieved"] / ceil["achieved"], 4)
        log(f"read ceiling: {ceil['mean_us']} us for {ceil['bytes_per_launch']} B, {ceil['achieved']} GB/s; "
            f"{ceil['achieved_one_launch']} GB/s reading {ceil['achieved_one_launch_of']} B in one launch")
    rows = None
    if not args.no_rows:
        t0 = time.time()
        g_rows, g_agg = gemv_sweep_rows()
        for r in g_rows:
            log(f"gemv {r['shape']}: {r['mean_us']} us, {r['achieved']} GB/s ({r['frac']:.3f}), "
                f"err {r['normwise_err_vs_oracle']:.1e}, oracle {r['oracle_gbs']} GB/s")
        log(f"gemv sweep aggregate: {g_agg['achieved']} GB/s ({g_agg['frac']:.3f})")
        b_rows = gemv_batch_rows()
        for r in b_rows:
            log(f"gemv batch {r['batch']} {r['shape']}: {r['mean_us']} us, {r['achieved']} GB/s "
                f"({r['frac']:.3f}), {r['vectors_per_s']:.0f} vectors/s, err {r['normwise_err_vs_oracle']:.1e}")
        x_row = experts_row()
        log(f"gemv experts {x_row['shape']}: {x_row['mean_us']} us, {x_row['achieved']} GB/s "
            f"({x_row['frac']:.3f}), err {x_row['normwise_err_vs_oracle']:.1e}")
        a_rows = attention_rows()
        a_rows += attention_rows(kv8=True)
        for r in a_rows:
            log(f"attention {r['case']} {r['kv']}: {r['mean_us']} us, {r['achieved']} GB/s "
                f"({r['frac']:.3f}), err {r['normwise_err_vs_oracle']:.1e}, oracle {r['oracle_s']} s")
        bd_rows = batch_decode_rows(mi, tuple(int(b) for b in args.batch_sizes.split(",")))
        d06 = decode_row("qwen3-0.6b") if args.config != "qwen3-0.6b" else None
        if d06:
            log(f"decode {d06['workload']}: {d06['tok_s']} tok/s ({d06['step_roofline']['frac']:.3f})")
        rows = {"gemv_sweep": g_rows, "gemv_sweep_aggregate": g_agg, "gemv_batch": b_rows,
                "gemv_experts": x_row,
                "attention": a_rows,
                "prefill": pf_row,
                "decode_batch": bd_rows,
                "decode_qwen3_0.6b": d06}
        log(f"row legs {time.time() - t0:.1f}s")
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(mi, t_pos0, toks_host)
        log(f"cpu baseline: {cpu['value']} tok/s on {cpu['cores']} threads")

    out = {
        "metric": "decode tok/s (batch 1) at Qwen3-8B shape; q4_0 GEMV GB/s as % of HBM peak",
        "value": round(tok_s, 2), "unit": "tok/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "q4_0/f32",
        "data": "synthetic (seeded N(0,0.02) weights quantised to q4_0, random prompt)",
        "config": {"workload": f"{s.name} batch-1 greedy decode, positions {pos}..{pos + args.steps - 1} "
                               f"after a {P}-token sequential-decode prefill",
                   "layers": s.layers, "hidden": s.hidden, "heads": f"{s.n_heads}/{s.n_kv}",
                   "head_dim": s.head_dim, "intermediate": s.intermediate, "vocab": s.vocab,
                   "kv": ("paged " if s.kv_paged else "contiguous ")
                         + ("fp8 e4m3 (k_scale 0.5, v_scale 0.125)" if args.kv_fp8 else "f16")
                         + (", block 16, shuffled table" if s.kv_paged else ""),
                   "batch": 1, "parallelism": "single GPU",
                   "kernels": "one persistent launch per layer" if args.layer_kernel else "five per layer"},
        "step_roofline": {"bound": "hbm", "achieved": round(step_gbs, 1), "peak": HBM_PEAK_GBS,
                          "unit": "GB/s", "frac": round(step_gbs / HBM_PEAK_GBS, 4),
                          "bytes_per_step": round(mean_bytes)},
        "roofline": roof,
        "cpu_baseline": cpu,
        "rows": rows,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
