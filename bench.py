#!/usr/bin/env python3
"""Benchmark: one decode step of KV4-RL attention on one MI355X.

A step is the whole hot path over the Qwen3-8B-shaped batch (1,024 sequences,
32 query / 8 KV heads, head_dim 128, 256-token prompts shared per group of 8,
lognormal responses with mean 2k capped at 16,384): kv4_append of one new
token per sequence, then kv4_decode_attention.  Inputs are synthetic, seeded
and already resident in HBM when timing starts.

Prints one JSON line.  `value` is context tokens per second (sum of the
sequences' context lengths / step time).  `roofline` is for the decode call
(work-list + attention + merge kernels, timed with HIP events on the stream
they run on) against the 8 TB/s HBM peak, with the algorithmic bytes of the
decode.  `cpu_baseline` times the CPU oracle on a bounded sample of the same
workload.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--variants] [--no-cpu]
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
CFG_IDX = 2


def algorithmic_bytes(wl, fmt):
    """Bytes the decode must move for this workload (unique shared pages once).

    Per (position, kv head): INT4 middle 144 B (64+64 code bytes, 8+8 scale
    bytes at head_dim 128), INT8 protected 260 B, kv8 260 B, bf16 512 B.
    Plus q and out (bf16), lse (fp32), one 4-byte page-table entry per page
    read and one seq_len per sequence.
    """
    cfg = wl.cfg
    H, D, Hq = cfg.num_kv_heads, cfg.head_dim, cfg.num_q_heads
    L = wl.lengths.astype(np.int64)
    B = L.size
    S, R = wl.layout.n_sink, wl.layout.n_recent
    int4_row = 2 * (D // 2) + 2 * 2 * (D // 32)
    int8_row = 2 * D + 4
    bf16_row = 4 * D
    if fmt == 0:
        prot = np.minimum(L, S + R)
        per_seq = (L - prot) * int4_row + prot * int8_row
        shared_mid = 0
        if cfg.group > 1:
            # prompt positions [S, prompt) are INT4 middle rows shared by the group
            p_mid = max(0, cfg.prompt_len - S)
            shared_mid = (B - (B + cfg.group - 1) // cfg.group) * p_mid * int4_row
        kv = H * (per_seq.sum() - 0) - H * shared_mid
    else:
        row = int8_row if fmt == 1 else bf16_row
        shared = 0
        if cfg.group > 1:
            shared = (B - (B + cfg.group - 1) // cfg.group) * cfg.prompt_len * row
        kv = H * (L.sum() * row) - H * shared
    pages = ((L + 15) // 16).sum()
    other = B * Hq * D * 2 * 2 + B * Hq * 4 + pages * 4 + B * 4
    return int(kv + other)


def time_steps(wl, steps, warmup, append=True):
    import torch

    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        if append:
            wl.step_append()
        wl.decode()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for a, b, c in ev:
        a.record(stream)
        if append:
            wl.step_append()
        b.record(stream)
        wl.decode()
        c.record(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    app = np.array([a.elapsed_time(b) for a, b, _ in ev])
    dec = np.array([b.elapsed_time(c) for _, b, c in ev])
    return total_ms / steps, app, dec


def cpu_baseline(wl, budget_s=12.0, max_seqs=256):
    """The oracle, untuned, on a bounded sample of the same workload."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import oracle
    import parity_util as pu

    oracle.build(force=False)
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    rng = np.random.default_rng(123)
    order = rng.permutation(wl.lengths.size)
    n = 8
    spent = 0.0
    rate = None
    used = 0
    while True:
        sample = np.sort(order[:n])
        ocache, pt, lens = pu.oracle_cache_for(wl, sample)
        q = np.ascontiguousarray(wl.host_q()[sample])
        # the step: append the last token of each sampled sequence, then decode
        k_last = np.stack([wl.host_tokens(int(b))[0][-1] for b in sample])
        v_last = np.stack([wl.host_tokens(int(b))[1][-1] for b in sample])
        cu = np.arange(len(sample) + 1, dtype=np.int32)
        t = time.perf_counter()
        oracle.append(ocache, pt, lens, None, k_last, v_last, cu)
        oracle.decode(ocache, pt, lens, None, q, 1.0, nthreads=threads)
        dt = time.perf_counter() - t
        spent += dt
        rate = float(lens.sum()) / dt
        used = len(sample)
        if dt > budget_s / 4 or n >= max_seqs or spent > budget_s:
            break
        n = min(max_seqs, n * 4)
    return {"value": rate, "unit": "ctx tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{used} sequences of the same workload (sum of contexts "
                      f"{int(wl.lengths[np.sort(order[:used])].sum())} tokens): oracle append of one "
                      f"token each + fp64 decode, {threads} OpenMP threads"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--variants", action="store_true", help="also time kv8 / bf16 / plain INT4")
    ap.add_argument("--no-cpu", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)

    import torch

    import int4_kv_cache_amd as kv4
    from harness import build_config

    kv4.load()
    torch.cuda.set_device(0)
    print(f"[bench] building config {CFG_IDX} (kv4) ...", file=sys.stderr, flush=True)
    wl = build_config(CFG_IDX, kv4.FMT_KV4, keep_inputs=not args.no_cpu)
    ctx = int(wl.lengths.sum())
    print(f"[bench] built: batch {wl.lengths.size}, ctx tokens {ctx}", file=sys.stderr, flush=True)
    ms, app, dec = time_steps(wl, args.steps, args.warmup)
    abytes = algorithmic_bytes(wl, 0)
    dec_ms = float(np.mean(dec))
    achieved = abytes / (dec_ms * 1e-3) / 1e9
    result = {
        "metric": "KV4 decode-attention ctx tokens/s (us/step and % HBM peak alongside), Qwen3-8B shape",
        "value": ctx / (ms * 1e-3),
        "unit": "ctx tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4/int8 codes, fp32 accumulate, bf16 out",
        "data": "synthetic (seeded)",
        "config": {"workload": "qwen3-8b-layer-b1024: 1024 seqs (128 groups x 8, shared 256-token "
                               "prompt), lognormal responses mean 2k cap 16384, Hq 32 / Hkv 8 / D 128, "
                               "16 sinks + 128 recent INT8",
                   "global_batch": int(wl.lengths.size), "ctx_tokens": ctx,
                   "append_us": float(np.mean(app)) * 1e3, "decode_us": dec_ms * 1e3,
                   "decode_us_median": float(np.median(dec)) * 1e3},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "kv4_decode_attention (worklist + attention + merge)",
                     "algorithmic_bytes": abytes},
    }
    if args.variants:
        var = {}
        for fmt, name, S, R in ((kv4.FMT_KV8, "kv8", 0, 0), (kv4.FMT_BF16, "bf16", 0, 0),
                                (kv4.FMT_KV4, "int4_plain", 0, 0)):
            w2 = build_config(CFG_IDX, fmt, n_sink=S, n_recent=R)
            _, _, d2 = time_steps(w2, max(5, args.steps // 2), 3, append=False)
            b2 = algorithmic_bytes(w2, fmt)
            var[name] = {"decode_us": float(np.mean(d2)) * 1e3,
                         "hbm_frac": b2 / (float(np.mean(d2)) * 1e-3) / 1e9 / HBM_PEAK_GBS}
            del w2
            torch.cuda.empty_cache()
        result["variants"] = var
    if not args.no_cpu:
        print("[bench] cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
