"""GPU parity: libkv4 (through the C ABI) against the CPU oracle.

Bit-exact cache bytes (codes, scales, side-cache rows); decode output within
rel-L2 1e-3 (vs the bf16-rounded oracle), max-abs 1e-2 (vs fp64) and lse
within 1e-4, on the same seeded inputs.
"""
import numpy as np
import pytest

import parity_util as pu

pytestmark = pytest.mark.gpu


def _run(kv4, wl):
    import torch

    wl.decode()
    torch.cuda.synchronize()


def _check_all(wl, sample=None, nthreads=0):
    sample = np.arange(wl.lengths.size) if sample is None else np.asarray(sample)
    ocache, pt, lens = pu.compare_bytes(wl, sample)
    m = pu.decode_metrics(wl, sample, ocache, pt, lens, nthreads=nthreads)
    print(f"\nparity {wl.cfg.name} fmt={wl.fmt} n={m['n']}: rel_l2={m['rel_l2']:.3e} "
          f"max_abs={m['max_abs']:.3e} lse={m['lse_abs']:.3e} rel_l2_vs_fp64={m['rel_l2_vs_fp64']:.3e}",
          flush=True)
    pu.assert_within(m)
    return m


@pytest.mark.parametrize("fmt", [0, 1, 2], ids=["kv4", "kv8", "bf16"])
def test_config0_full(kv4, fmt):
    from harness import build_from_host

    wl = build_from_host(0, fmt)
    _run(kv4, wl)
    _check_all(wl)


def test_config0_plain_int4(kv4):
    from harness import build_from_host

    wl = build_from_host(0, kv4.FMT_KV4, n_sink=0, n_recent=0)
    _run(kv4, wl)
    _check_all(wl)


EDGE_LENGTHS = [0, 1, 2, 3, 4, 5, 15, 16, 17, 19, 20, 21, 31, 32, 33, 36, 37, 48, 300, 517, 1023, 1025]


@pytest.mark.parametrize("fmt", [0, 1, 2], ids=["kv4", "kv8", "bf16"])
def test_edge_lengths_and_slot_permutation(kv4, fmt):
    from harness import build_from_host

    wl = build_from_host(0, fmt, lengths=EDGE_LENGTHS, slot_perm_seed=3)
    _run(kv4, wl)
    _check_all(wl)
    import torch

    out = wl.out.float().cpu().numpy()
    assert np.all(out[0] == 0), "empty context decodes to zero"
    assert np.all(np.isneginf(wl.lse.cpu().numpy()[0]))


@pytest.mark.parametrize("S,R", [(0, 16), (4, 0), (16, 128), (144, 0), (0, 144), (5, 7)])
def test_protection_widths(kv4, S, R):
    from harness import build_from_host

    wl = build_from_host(0, kv4.FMT_KV4, lengths=[1, 9, 150, 151, 160, 700, 2100], n_sink=S, n_recent=R)
    _run(kv4, wl)
    _check_all(wl)


def test_token_by_token_equals_bulk(kv4):
    """Calibration-free: appending one token per call gives the same bytes."""
    from harness import build_from_host

    lengths = [5, 37, 70]
    a = build_from_host(0, kv4.FMT_KV4, lengths=lengths)
    b = build_from_host(0, kv4.FMT_KV4, lengths=lengths, token_by_token=True)
    assert np.array_equal(a.cache.pages.cpu().numpy(), b.cache.pages.cpu().numpy())
    assert np.array_equal(a.cache.side.cpu().numpy(), b.cache.side.cpu().numpy())


@pytest.mark.parametrize("hq,hkv,d", [(32, 8, 128), (8, 8, 128), (16, 8, 64), (8, 1, 64), (16, 2, 128)])
def test_head_shapes(kv4, hq, hkv, d):
    """GQA group sizes 1..8 and both head dims, on host-drawn data."""
    import dataclasses

    import workloads.configs as wc
    from harness import build_from_host

    base = wc.CONFIGS[0]
    cfg = dataclasses.replace(base, idx=90, name=f"shape-{hq}-{hkv}-{d}", num_q_heads=hq,
                              num_kv_heads=hkv, head_dim=d, n_sink=16, n_recent=128, n_outlier=6)
    wc.CONFIGS[90] = cfg
    try:
        for fmt in (0, 1, 2):
            wl = build_from_host(90, fmt, lengths=[1, 160, 1300, 77])
            _run(kv4, wl)
            _check_all(wl)
    finally:
        del wc.CONFIGS[90]


def test_golden_quantizer_cases_on_gpu(kv4):
    """The hand-worked quantizer cases, appended by the GPU."""
    import os

    import torch

    import int4_kv_cache_amd as lib
    from test_oracle_quantizer import CASES

    for c in CASES:
        D = 64 if c["qmax"] == 7 else c["n"]
        fmt = lib.FMT_KV4 if c["qmax"] == 7 else lib.FMT_KV8
        lay = lib.make_layout(1, 1, D, 0, 0)
        cache = lib.alloc_cache(fmt, lay, 1, 1)
        k = np.zeros((1, 1, D), dtype=np.uint16)
        k[0, 0, :len(c["x"])] = c["x"]
        kt = torch.as_tensor(k.view(np.int16), device="cuda").view(torch.bfloat16)
        i32 = lambda a: torch.as_tensor(np.asarray(a, np.int32), device="cuda")
        lib.append(cache, lib.Batch(i32([[0]]), i32([1])), kt, torch.zeros_like(kt), i32([0, 1]))
        got = cache.pages.cpu().numpy()
        assert got[:len(c["packed"])].tolist() == c["packed"], c["id"]
        off = 16 * D if fmt == lib.FMT_KV4 else 32 * D
        assert int(got[off]) | (int(got[off + 1]) << 8) == c["scale"], c["id"]


def test_golden_layout_cases_on_gpu(kv4):
    """The hand-worked byte-layout cases (K and V codes and scales of INT4
    pages, INT8 pages, the INT8 side tile and bf16 pages), appended by the GPU."""
    import torch

    import int4_kv_cache_amd as lib
    from test_oracle_layout_golden import CASES, case_inputs, expected_buffer

    i32 = lambda a: torch.as_tensor(np.asarray(a, np.int32), device="cuda")
    for c in CASES:
        fmt = {0: lib.FMT_KV4, 1: lib.FMT_KV8, 2: lib.FMT_BF16}[c["fmt"]]
        lay = lib.make_layout(1, 1, c["D"], c["S"], c["R"])
        cache = lib.alloc_cache(fmt, lay, 1, 1)
        k, v = case_inputs(c)
        kt = torch.as_tensor(k.view(np.int16), device="cuda").view(torch.bfloat16)
        vt = torch.as_tensor(v.view(np.int16), device="cuda").view(torch.bfloat16)
        lib.append(cache, lib.Batch(i32([[0]]), i32([16])), kt, vt, i32([0, 16]))
        buf = cache.pages if c["area"] == "page" else cache.side
        got = buf.cpu().numpy()
        want = expected_buffer(c, got.size)
        bad = np.flatnonzero(got != want)
        assert bad.size == 0, f"{c['id']}: bytes differ at {bad[:8].tolist()}"


def test_config1_sampled(kv4):
    from harness import build_config

    wl = build_config(1, kv4.FMT_KV4, keep_inputs=True)
    wl.step_append()
    _run(kv4, wl)
    order = np.argsort(wl.lengths)
    sample = np.unique(np.concatenate([order[:4], order[-4:], np.arange(0, 128, 9)]))
    _check_all(wl, sample)


def _bench_step(wl):
    """One decode step exactly as bench.py times it: the fused append + plan
    launch, then ATTEND, then MERGE (GpuWorkload.step_launches)."""
    import torch

    for launch in wl.step_launches():
        launch()
    torch.cuda.synchronize()


def _config2_sample(wl, seed):
    order = np.argsort(wl.lengths)
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([order[:6], order[-6:], rng.choice(wl.lengths.size, 20, replace=False),
                                     np.arange(8)]))   # a whole prompt group


def test_config2_full_size_bench_launch(kv4):
    """Config 2 at full size through the benchmark's own launch sequence
    (kv4_append_decode_phases with the plan, then ATTEND and MERGE),
    checked on sampled sequences: their page and side bytes, including the
    step token the fused launch appended, and their outputs."""
    from harness import build_config

    wl = build_config(2, kv4.FMT_KV4, keep_inputs=True)
    _bench_step(wl)
    chunk = wl.plan_chunk_pages()
    print(f"\nconfig 2 plan: {chunk}-page chunks", flush=True)
    assert chunk > 64, "the bench workload runs the two-page-ids-per-lane path"
    _check_all(wl, _config2_sample(wl, 0))


@pytest.mark.parametrize("fmt,S,R", [(1, 0, 0), (2, 0, 0), (0, 0, 0)], ids=["kv8", "bf16", "int4_plain"])
def test_config2_full_size_variants(kv4, fmt, S, R):
    """The reference variants of the precision ablation at the config-2 batch
    (1,024 sequences, chunks of the largest size, 128 pages), through the benchmark's launch
    sequence, against the oracle on sampled sequences."""
    from harness import build_config

    wl = build_config(2, fmt, keep_inputs=True, n_sink=S, n_recent=R)
    _bench_step(wl)
    chunk = wl.plan_chunk_pages()
    print(f"\nconfig 2 fmt={fmt} S={S} R={R}: {chunk}-page chunks", flush=True)
    assert chunk > 64
    _check_all(wl, _config2_sample(wl, 1 + fmt))


@pytest.mark.parametrize("fmt", [0, 1, 2], ids=["kv4", "kv8", "bf16"])
def test_head_dim64_long_chunks(kv4, fmt):
    """Head_dim 64 at the config-2 batch: enough pages that the plan cuts
    chunks of more than 64 pages (two page ids per lane) for every format."""
    import dataclasses

    import workloads.configs as wc
    from harness import build_config

    cfg = dataclasses.replace(wc.CONFIGS[2], idx=93, name="config2-d64", head_dim=64)
    wc.CONFIGS[93] = cfg
    try:
        wl = build_config(93, fmt, keep_inputs=True)
        _bench_step(wl)
        chunk = wl.plan_chunk_pages()
        print(f"\nhead_dim 64 fmt={fmt}: {chunk}-page chunks", flush=True)
        assert chunk > 64
        _check_all(wl, _config2_sample(wl, 7))
    finally:
        del wc.CONFIGS[93]


@pytest.mark.parametrize("int8_query", [False, True], ids=["bf16q", "int8q"])
def test_shared_prompt_pages(kv4, int8_query):
    """Two prompt groups of 8 at the config-2 shapes, with lengths that put
    the end of the INT4 region before, at and after the end of the shared
    prompt pages (an odd number of them).  Shared pages and private pages are
    read on different load paths; every sequence is checked in full."""
    from harness import build_config

    lengths = np.array([257, 300, 383, 384, 385, 512, 529, 1000,
                        400, 700, 1500, 2049, 271, 640, 900, 3000], dtype=np.int32)
    wl = build_config(2, kv4.FMT_KV4, keep_inputs=True, lengths=lengths, int8_query=int8_query)
    wl.step_append()
    _run(kv4, wl)
    _check_all(wl)


# ---- the integer query-key path (KV4_LAYOUT_INT8_QUERY) ----------------------
def test_int8_query_config0_and_edges(kv4):
    from harness import build_from_host

    wl = build_from_host(0, kv4.FMT_KV4, int8_query=True)
    _run(kv4, wl)
    _check_all(wl)
    wl = build_from_host(0, kv4.FMT_KV4, lengths=EDGE_LENGTHS, slot_perm_seed=3, int8_query=True)
    _run(kv4, wl)
    _check_all(wl)
    wl = build_from_host(0, kv4.FMT_KV4, n_sink=0, n_recent=0, int8_query=True)
    _run(kv4, wl)
    _check_all(wl)


@pytest.mark.parametrize("hq,hkv,d", [(32, 8, 128), (8, 8, 128), (16, 8, 64), (8, 1, 64), (16, 2, 128)])
def test_int8_query_head_shapes(kv4, hq, hkv, d):
    import dataclasses

    import workloads.configs as wc
    from harness import build_from_host

    base = wc.CONFIGS[0]
    cfg = dataclasses.replace(base, idx=91, name=f"q8-shape-{hq}-{hkv}-{d}", num_q_heads=hq,
                              num_kv_heads=hkv, head_dim=d, n_sink=16, n_recent=128, n_outlier=6)
    wc.CONFIGS[91] = cfg
    try:
        wl = build_from_host(91, kv4.FMT_KV4, lengths=[1, 160, 1300, 77], int8_query=True)
        _run(kv4, wl)
        _check_all(wl)
    finally:
        del wc.CONFIGS[91]


def test_int8_query_config2_full_size(kv4):
    from harness import build_config

    wl = build_config(2, kv4.FMT_KV4, keep_inputs=True, int8_query=True)
    wl.step_append()
    _run(kv4, wl)
    order = np.argsort(wl.lengths)
    rng = np.random.default_rng(1)
    sample = np.unique(np.concatenate([order[:6], order[-6:], rng.choice(1024, 20, replace=False)]))
    _check_all(wl, sample)
