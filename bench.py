#!/usr/bin/env python3
"""Benchmark: one decode step of KV4-RL attention on one MI355X.

A step is the whole hot path over the Qwen3-8B-shaped batch (1,024 sequences,
32 query / 8 KV heads, head_dim 128, 256-token prompts shared per group of 8,
lognormal responses with mean 2k capped at 16,384): kv4_append of one new
token per sequence, then kv4_decode_attention.  Inputs are synthetic, seeded
and already resident in HBM when timing starts.

Prints one JSON line.  `value` is context tokens per second (sum of the
sequences' context lengths / step time).  The decode runs as its three phases
(kv4_decode_phases: plan, attend, merge); in the timed region the attention
launch is bracketed by HIP events on the stream it runs on, and a second pass
of the same steps times every phase.  `roofline` is for the dominant kernel, the attention
kernel of the ATTEND phase, against the 8 TB/s HBM peak with its algorithmic
bytes; `traffic` is the HBM bytes per launch from the committed rocprofv3
counter runs (null once the kernel sources differ from the ones measured).
`cpu_baseline` times the CPU oracle on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-variants] [--no-cpu] [--mq T]
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


def attend_bytes(wl, fmt):
    """Algorithmic bytes credited to the ATTEND phase (the attention kernel):
    the decode's bytes less the bf16 output and the lse, which the merge
    writes for sequences split over several work items (0.3% of the total at
    the Qwen3-8B batch; leaving all of it out under-counts slightly)."""
    cfg = wl.cfg
    B = wl.lengths.size
    return int(algorithmic_bytes(wl, fmt) - B * cfg.num_q_heads * (cfg.head_dim * 2 + 4))


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attention_kv4_qwen3-8b-b1024_traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "int4_kv_cache_amd", "csrc", f)
                  for f in ("decode.hip", "kv4_common.h", "kv4_launch.h")]


def kernel_source_hash():
    """sha256 of the kernel sources with comments and blank space removed, so
    an edit of a comment does not discard a measurement of the same code."""
    import hashlib
    import re

    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f) as fh:
            src = fh.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per ATTEND launch from the committed rocprofv3 counter runs,
    or None when the kernel sources changed since they were taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def settle(step, min_s=2.0, max_s=12.0, window=100):
    """Run `step` in windows of `window` calls, timed with HIP events, until at
    least `min_s` seconds have passed and two windows in a row agree within
    1%, or `max_s` seconds.  The GPU raises its clocks over the first second
    or so of sustained load (a timed region that starts on a cold GPU ran the
    attention kernel about 10% slower), so this runs before the requested
    warm-up steps whatever their number.  Returns (calls, seconds, last
    window's ms per call)."""
    import torch

    stream = torch.cuda.current_stream()
    t0 = time.perf_counter()
    calls, prev, last = 0, None, None
    while True:
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(window):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        calls += window
        last = e0.elapsed_time(e1) / window
        el = time.perf_counter() - t0
        if el >= max_s or (el >= min_s and prev is not None and abs(last - prev) <= 0.01 * prev):
            return calls, el, last
        prev = last


def time_steps(wl, steps, warmup, settle_s=2.0):
    """Time `steps` decode steps after the clock-settling run and `warmup`
    untimed steps.

    A step is GpuWorkload.step_launches(): the append of one token per
    sequence with the plan in the same launch (kv4_append_decode_phases), then
    ATTEND, then MERGE, on one stream.  In the timed region only the attention
    launch is bracketed by HIP events on that stream (every event record
    costs the stream 2-3 us).  A second pass of the same steps puts an event
    between every launch; every per-phase figure comes from that pass.
    Returns (mean ms per step of the timed region, attend ms per step of the
    timed region, per-phase ms arrays of the second pass, settle record).
    """
    import torch

    stream = torch.cuda.current_stream()
    launches = wl.step_launches()

    def step():
        for launch in launches:
            launch()

    n_settle, s_settle, ms_settle = settle(step, min_s=settle_s)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    plan, attend, merge = launches
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for e in ev:
        plan()
        e[0].record(stream)
        attend()
        e[1].record(stream)
        merge()
    t1.record(stream)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    att = np.array([e[0].elapsed_time(e[1]) for e in ev])
    # phase pass: an event between every launch
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for e in ev:
        e[0].record(stream)
        plan()
        e[1].record(stream)
        attend()
        e[2].record(stream)
        merge()
        e[3].record(stream)
    torch.cuda.synchronize()
    ph = {name: np.array([e[i].elapsed_time(e[i + 1]) for e in ev])
          for i, name in enumerate(("append_plan", "attend", "merge"))}
    ph["step"] = np.array([e[0].elapsed_time(e[3]) for e in ev])
    return total_ms / steps, att, ph, {"steps": n_settle, "s": round(s_settle, 2),
                                       "last_window_ms_per_step": ms_settle}


MFMA_BF16_PEAK_TFLOPS = 2500.0


def time_multi_query(wl, T, steps, warmup, decode_bytes, step_us):
    """kv4_decode_attention_mq with T query tokens per sequence over the
    workload's cache as it stands (the last T positions are the queries),
    timed with HIP events around each call (plan + attend + merge; the
    attention kernel is all but a few tens of microseconds of it).

    Two rooflines.  HBM: the single-token decode's algorithmic bytes (every
    cache byte once) plus the q / out / lse of the T - 1 extra queries.
    Matrix cores: the useful flops, 4 * head_dim per (query, query head,
    position it sees) -- 2 * D for q.k and 2 * D for p.v -- against the
    2.5 PFLOP/s dense bf16 peak.  The multi-column kernel is bound by neither:
    it is bound by instruction issue (conversions, scales and the softmax on
    the vector ALU next to the MFMAs), so both fractions are low."""
    import torch

    import int4_kv_cache_amd as kv4
    from workloads.gen import device_queries

    cfg = wl.cfg
    B = int(wl.lengths.size)
    q = device_queries(cfg, 0, B, "cuda", n_queries=T)
    out = torch.empty((B, T, cfg.num_q_heads, cfg.head_dim), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, T, cfg.num_q_heads), dtype=torch.float32, device="cuda")
    ws = torch.empty(kv4.workspace_bytes(wl.layout, B * T, wl.alloc.page_table.shape[1]),
                     dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def call():
        kv4.decode_mq(wl.cache, wl.batch, q, T, out, lse, ws)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for e in ev:
        e[0].record(stream)
        call()
        e[1].record(stream)
    torch.cuda.synchronize()
    per = np.array([e[0].elapsed_time(e[1]) for e in ev]) * 1e3
    us = float(per.mean())
    extra = (T - 1) * B * cfg.num_q_heads * (cfg.head_dim * 4 + 4)
    nbytes = decode_bytes + extra
    L = wl.lengths.astype(np.int64)
    seen = sum(np.maximum(L - T + t + 1, 0).sum() for t in range(T))
    flops = float(seen) * cfg.num_q_heads * 4 * cfg.head_dim
    tflops = flops / (us * 1e-6) / 1e12
    del q, out, lse, ws
    torch.cuda.empty_cache()
    return {"T": T, "us": us, "us_min": float(per.min()), "query_tokens_per_s": B * T / (us * 1e-6),
            "hbm_frac": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, "algorithmic_bytes": int(nbytes),
            "roofline_mfma": {"bound": "issue", "achieved": tflops, "peak": MFMA_BF16_PEAK_TFLOPS,
                              "unit": "TFLOP/s", "frac": tflops / MFMA_BF16_PEAK_TFLOPS,
                              "algorithmic_flops": flops},
            "vs_T_single_token_steps": us / (T * step_us),
            "note": "plan + attend + merge; at head_dim 128 on INT4 pages one unit serves 16 / G "
                    "queries (the multi-column kernel), otherwise each query reads the cache itself"}


def capacity(budget_gb=240.0, layers=36, repeats=64):
    """Concurrent sequences whose cache fits a fixed budget (kv4_cache_capacity,
    host arithmetic): Qwen3-8B attention (36 layers, Hkv 8, D 128) with the
    config-2 length distribution tiled `repeats` times.  240 GB is the MI355X's
    288 GB less the bf16 weights (about 16 GB) and about 10% headroom."""
    import int4_kv_cache_amd as kv4
    from workloads import context_lengths, get_config

    cfg = get_config(CFG_IDX)
    lengths = np.tile(context_lengths(cfg), repeats)
    budget = int(budget_gb * 1e9)
    out = {}
    for name, fmt, S, R in (("bf16", kv4.FMT_BF16, 0, 0), ("kv8", kv4.FMT_KV8, 0, 0),
                            ("int4_plain", kv4.FMT_KV4, 0, 0), ("kv4_rl", kv4.FMT_KV4, cfg.n_sink, cfg.n_recent)):
        lay = kv4.make_layout(cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, S, R)
        out[name] = kv4.cache_capacity(lay, fmt, layers, lengths, budget)[1]
    return {"budget_gb": budget_gb, "layers": layers, "lengths": "config-2 distribution (mean %.0f)" % lengths.mean(),
            "sequences": out, "vs_bf16": {k: out[k] / out["bf16"] for k in out}}


def cpu_baseline(wl, budget_s=12.0, max_seqs=256, threads=None):
    """The oracle, untuned, on a bounded sample of the same workload, with
    `threads` OpenMP threads (default: OMP_NUM_THREADS, else every core)."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import oracle
    import parity_util as pu

    oracle.build(force=False)
    if threads is None:
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
        last = [wl.host_tokens(int(b)) for b in sample]
        k_last = np.stack([k[-1] for k, _ in last])
        v_last = np.stack([v[-1] for _, v in last])
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


def read_probe_gbs(nbytes=4 << 30, reps=5):
    """Achievable streaming read bandwidth: kv4_hbm_read_probe over `nbytes`
    (128-bit nontemporal loads, contiguous per wave), HIP events."""
    import torch

    import int4_kv_cache_amd as kv4

    buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(kv4.probe_blocks(), dtype=torch.int32, device="cuda")
    for _ in range(2):
        kv4.hbm_read_probe(buf, sink)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        kv4.hbm_read_probe(buf, sink)
    e1.record()
    torch.cuda.synchronize()
    gbs = nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del buf, sink
    torch.cuda.empty_cache()
    return gbs


def copy_calibration(nbytes=1 << 30):
    """A plain copy kernel of known size: each launch reads and writes
    `nbytes`, so FETCH_SIZE / WRITE_SIZE of its dispatches give the factor from
    counter KiB to HBM bytes."""
    import torch

    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": nbytes, "launches": 3}), flush=True)


def run_layers(args):
    """The 36-layer decode step (config 3): one plan, then attend + merge for
    every layer (each its own INT4 pool and INT8 side cache), timed with HIP
    events around each phase.  Prints one JSON line."""
    import torch

    import int4_kv_cache_amd as kv4
    from harness import build_layers

    kv4.load()
    torch.cuda.set_device(0)
    print("[bench] building config 3 (36 layers) ...", file=sys.stderr, flush=True)
    t = time.time()
    wl = build_layers(3, kv4.FMT_KV4,
                      progress=lambda l: print(f"[bench] layer {l} built", file=sys.stderr, flush=True))
    print(f"[bench] built in {time.time() - t:.1f} s", file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream()
    nl = wl.n_layers
    for _ in range(args.warmup):
        wl.step()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2 + 2 * nl)] for _ in range(args.steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for e in ev:
        e[0].record(stream)
        wl.plan()
        e[1].record(stream)
        for l in range(nl):
            kv4.decode_phases(wl.caches[l], wl.batch, wl.qs[l], wl.out[l], wl.lse[l], wl.workspace,
                              kv4.PHASE_ATTEND)
            e[2 + 2 * l].record(stream)
            kv4.decode_phases(wl.caches[l], wl.batch, wl.qs[l], wl.out[l], wl.lse[l], wl.workspace,
                              kv4.PHASE_MERGE)
            e[3 + 2 * l].record(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    plan = np.array([e[0].elapsed_time(e[1]) for e in ev])
    att = np.array([[(e[1] if l == 0 else e[1 + 2 * l]).elapsed_time(e[2 + 2 * l]) for l in range(nl)]
                    for e in ev])
    mrg = np.array([[e[2 + 2 * l].elapsed_time(e[3 + 2 * l]) for l in range(nl)] for e in ev])
    view = wl.layer(0)
    layer_bytes = algorithmic_bytes(view, 0)
    att_bytes = attend_bytes(view, 0)
    ctx = int(wl.lengths.sum())
    att_ms = float(att.mean())
    achieved = att_bytes / (att_ms * 1e-3) / 1e9
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
        "dtype": "int4/int8 codes x bf16 q on bf16 MFMA, fp32 accumulate, bf16 out",
        "data": "synthetic (seeded)",
        "config": {"workload": "qwen3-8b-36-layers-b512: 36 layers x (Hq 32 / Hkv 8 / D 128), 512 seqs, "
                               "contexts uniform in [4096, 16600], 16 sinks + 128 recent INT8; step = one "
                               "plan + attend/merge of all 36 layers",
                   "global_batch": int(wl.lengths.size), "ctx_tokens": ctx, "layers": nl,
                   "plan_us": float(plan.mean()) * 1e3, "attend_us_per_layer": att_ms * 1e3,
                   "merge_us_per_layer": float(mrg.mean()) * 1e3,
                   "step_hbm_frac": nl * layer_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                   "step_algorithmic_bytes": nl * layer_bytes,
                   "resident_gb": sum(c.pages.numel() + (c.side.numel() if c.side is not None else 0)
                                      for c in wl.caches) / 1e9},
        "hbm_read_probe_gbs": read_probe_gbs(),
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "attention_kernel<kv4, 128> (the ATTEND phase), mean over the 36 layers",
                     "algorithmic_bytes": att_bytes},
    }
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the bf16 / kv8 / plain INT4 / integer-query variants on the same workload")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--config", type=int, default=CFG_IDX, choices=(2, 3),
                    help="2: one Qwen3-8B-shaped layer, B=1024 (the default line); 3: the 36-layer "
                         "decode step at B=512 (about 226 GB resident)")
    ap.add_argument("--mq", type=int, default=0, metavar="T",
                    help="also time the multi-query decode with T query tokens per sequence over "
                         "the same cache (kv4_decode_attention_mq)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy 3 times (scales the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this library is measured on one GPU; --gpus must be 1 (the path would shard over sequences or kv heads without exchange inside attention)"}))
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.config == 3:
        run_layers(args)
        return

    import torch

    import int4_kv_cache_amd as kv4
    from harness import build_config

    kv4.load()
    torch.cuda.set_device(0)
    print(f"[bench] building config {CFG_IDX} (kv4) ...", file=sys.stderr, flush=True)
    wl = build_config(CFG_IDX, kv4.FMT_KV4, keep_inputs=not args.no_cpu)
    ctx = int(wl.lengths.sum())
    print(f"[bench] built: batch {wl.lengths.size}, ctx tokens {ctx}", file=sys.stderr, flush=True)
    ms, att, ph, settled = time_steps(wl, args.steps, args.warmup)
    abytes = algorithmic_bytes(wl, 0)
    att_ms = float(np.mean(att))
    achieved = attend_bytes(wl, 0) / (att_ms * 1e-3) / 1e9
    us = {k: float(np.mean(v)) * 1e3 for k, v in ph.items()}
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
        "dtype": "int4/int8 codes x bf16 q on bf16 MFMA, fp32 accumulate, bf16 out",
        "data": "synthetic (seeded)",
        "config": {"workload": "qwen3-8b-layer-b1024: 1024 seqs (128 groups x 8, shared 256-token "
                               "prompt), lognormal responses mean 2k cap 16384, Hq 32 / Hkv 8 / D 128, "
                               "16 sinks + 128 recent INT8; step = append 1 token/seq + decode",
                   "global_batch": int(wl.lengths.size), "ctx_tokens": ctx,
                   "attend_us": att_ms * 1e3,
                   "attend_us_per_step": [round(float(x) * 1e3, 1) for x in att],
                   "attend_us_median": float(np.median(att)) * 1e3,
                   "phases_us": {"append_plan": us["append_plan"], "attend": us["attend"],
                                 "merge": us["merge"], "step": us["step"],
                                 "note": "one pass with an event between every launch (each record costs "
                                         "2-3 us); append_plan is the append of the step tokens with the "
                                         "plan in the same launch"},
                   "step_hbm_frac": abytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                   "decode_algorithmic_bytes": abytes,
                   "settle": dict(settled, note="clock-settling steps run before the warm-up steps")},
        "hbm_read_probe_gbs": read_probe_gbs(),
        "capacity": capacity(),
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(),
                     "kernel": "attention_kernel<kv4, 128> (the ATTEND phase)",
                     "algorithmic_bytes": attend_bytes(wl, 0)},
    }
    if not args.no_variants:
        # the reference kernels and plain INT4 on the same seeded workload
        # (config 4's formats), each timed like the KV4-RL step
        var = {}
        for fmt, name, S, R, q8 in ((kv4.FMT_BF16, "bf16", 0, 0, False), (kv4.FMT_KV8, "kv8", 0, 0, False),
                                    (kv4.FMT_KV4, "int4_plain", 0, 0, False),
                                    (kv4.FMT_KV4, "kv4_rl_int8_query", None, None, True)):
            print(f"[bench] variant {name} ...", file=sys.stderr, flush=True)
            w2 = build_config(CFG_IDX, fmt, n_sink=S, n_recent=R, int8_query=q8)
            ms2, att2, ph2, _ = time_steps(w2, args.steps, 3, settle_s=0.5)
            b2 = algorithmic_bytes(w2, fmt)
            a2 = float(np.mean(att2))
            var[name] = {"step_us": ms2 * 1e3, "attend_us": a2 * 1e3,
                         "step_hbm_frac": b2 / (ms2 * 1e-3) / 1e9 / HBM_PEAK_GBS,
                         "attend_hbm_frac": attend_bytes(w2, fmt) / (a2 * 1e-3) / 1e9 / HBM_PEAK_GBS}
            del w2
            torch.cuda.empty_cache()
        var["kv4_rl"] = {"step_us": ms * 1e3, "attend_us": att_ms * 1e3,
                         "step_hbm_frac": result["config"]["step_hbm_frac"],
                         "attend_hbm_frac": achieved / HBM_PEAK_GBS}
        for v in var.values():
            v["step_speedup_vs_bf16"] = var["bf16"]["step_us"] / v["step_us"]
        result["variants"] = var
    if args.mq > 0:
        result["multi_query"] = time_multi_query(wl, args.mq, max(10, args.steps // 2), 3, abytes, us["step"])
    if not args.no_cpu:
        print("[bench] cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(wl)
        one = cpu_baseline(wl, budget_s=8.0, threads=1)
        result["cpu_baseline"]["single_core"] = {"value": one["value"], "cores": 1, "sample": one["sample"]}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
