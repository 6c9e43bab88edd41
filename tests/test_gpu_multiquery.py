"""GPU parity of the multi-query decode (kv4_decode_attention_mq and the kv8 /
kvbf16 variants) against the oracle's multi-query decode on the same bytes.

Query t of sequence b sees the first seq_lens[b] - T + t + 1 positions of the
cache as it stands after the append (a reading of this library; the pages
describe the single-token step).  Bounds as in the single-token parity
tests: rel-L2 1e-3 against the bf16-rounded oracle, max-abs 1e-2 and lse
1e-4 against fp64.
"""
import numpy as np
import pytest

import oracle
import parity_util as pu
from workloads import get_config, host_queries

pytestmark = pytest.mark.gpu


def _run_mq(kv4, wl, T, seed_layer=0):
    import torch

    cfg = wl.cfg
    B = wl.lengths.size
    qh = host_queries(cfg, seed_layer, B, T)
    q = torch.from_numpy(qh.view(np.int16)).to("cuda").view(torch.bfloat16)
    out = torch.zeros((B, T, cfg.num_q_heads, cfg.head_dim), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((B, T, cfg.num_q_heads), dtype=torch.float32, device="cuda")
    mp = wl.alloc.page_table.shape[1]
    ws = torch.empty(kv4.workspace_bytes(wl.layout, B * T, mp), dtype=torch.uint8, device="cuda")
    kv4.decode_mq(wl.cache, wl.batch, q, T, out, lse, ws)
    torch.cuda.synchronize()
    og = pu.bf16_bits_to_f64(out.view(torch.int16).cpu().numpy())
    lg = lse.cpu().numpy().astype(np.float64)
    return qh, og, lg


def _check(kv4, wl, T, label):
    sample = np.arange(wl.lengths.size)
    ocache, pt, lens = pu.compare_bytes(wl, sample)
    qh, og, lg = _run_mq(kv4, wl, T)
    q_int8 = bool(wl.layout.flags & 2)  # the integer-query layout flag
    out64, lse64, gap = oracle.decode_mq(ocache, pt, lens, None, qh, T, q_int8=q_int8)
    m = pu.metrics_from(og, lg, out64, lse64, gap)
    print(f"\nmulti-query {label} T={T}: rel_l2={m['rel_l2']:.3e} max_abs={m['max_abs']:.3e} "
          f"lse={m['lse_abs']:.3e}", flush=True)
    pu.assert_within(m)
    # queries that see no position
    for b, N in enumerate(wl.lengths):
        for t in range(T):
            if N - T + t + 1 <= 0:
                assert np.all(og[b, t] == 0.0) and np.all(np.isneginf(lg[b, t]))
    return m


@pytest.mark.parametrize("fmt", [0, 1, 2], ids=["kv4", "kv8", "bf16"])
@pytest.mark.parametrize("T", [1, 3, 8])
def test_multiquery_small(kv4, fmt, T):
    """D = 64, 4 sinks + 16 recent; lengths below, at and across the
    protected bounds and shorter than T."""
    from harness import build_from_host

    lengths = np.array([300, 517, 5, 21, 16, 20, 37, 2, 33, 100], dtype=np.int32)
    wl = build_from_host(0, fmt, lengths=lengths)
    _check(kv4, wl, T, f"cfg0 fmt={fmt}")


@pytest.mark.parametrize("T", [5, 9, 20])
def test_multiquery_more_queries_than_ring(kv4, T):
    """T larger than the ring (R = 4): early queries end before the ring and
    read their recent positions from INT4."""
    from harness import build_from_host

    lengths = np.array([64, 29, 11, 90, 7], dtype=np.int32)
    wl = build_from_host(0, 0, lengths=lengths, n_sink=4, n_recent=4)
    _check(kv4, wl, T, "cfg0 S=4 R=4")


@pytest.mark.parametrize("T", [2, 4])
def test_multiquery_qwen_shapes(kv4, T):
    """Hq 32 / Hkv 8 / D 128 with 16 sinks + 128 recent; split sequences (the
    merge path) and a sequence within the protected set."""
    from harness import build_from_host

    lengths = np.array([2100, 700, 145, 1000, 290, 60], dtype=np.int32)
    wl = build_from_host(1, 0, lengths=lengths)
    _check(kv4, wl, T, "qwen shapes")


@pytest.mark.parametrize("T", [3, 5, 6, 12])
def test_multiquery_blocks_and_short_ring(kv4, T):
    """Qwen shapes with a ring of 8: blocks of four queries, partial last
    blocks, and queries whose view ends inside the INT4 region."""
    from harness import build_from_host

    lengths = np.array([1500, 333, 40, 12, 700], dtype=np.int32)
    wl = build_from_host(1, 0, lengths=lengths, n_sink=16, n_recent=8)
    _check(kv4, wl, T, "qwen shapes S=16 R=8")


@pytest.mark.parametrize("hq,hkv", [(8, 8), (16, 8), (8, 1), (4, 1)])
def test_multiquery_group_sizes(kv4, hq, hkv):
    """Head dim 128 with 1, 2, 8 and 4 query heads per kv head (16, 8, 2 and
    4 queries per block; the layout allows up to 8 per kv head)."""
    import dataclasses

    import workloads.configs as wc
    from harness import build_from_host

    base = wc.CONFIGS[1]
    cfg = dataclasses.replace(base, idx=91, name=f"mq-shape-{hq}-{hkv}", num_q_heads=hq, num_kv_heads=hkv)
    wc.CONFIGS[91] = cfg
    try:
        wl = build_from_host(91, 0, lengths=np.array([1, 160, 1300, 77], dtype=np.int32))
        for T in (3, 17):
            _check(kv4, wl, T, f"hq={hq} hkv={hkv}")
    finally:
        del wc.CONFIGS[91]


@pytest.mark.parametrize("T", [2, 5])
def test_multiquery_integer_query(kv4, T):
    """The integer-query layout with several queries (one query per unit on
    the integer path), Qwen shapes and the tiny shapes."""
    from harness import build_from_host

    wl = build_from_host(1, 0, lengths=np.array([700, 145, 1000, 60], dtype=np.int32), int8_query=True)
    _check(kv4, wl, T, "qwen shapes int8 query")
    wl = build_from_host(0, 0, lengths=np.array([300, 5, 21, 2], dtype=np.int32), int8_query=True)
    _check(kv4, wl, T, "cfg0 int8 query")


@pytest.mark.parametrize("S,R", [(16, 128), (0, 16), (5, 7), (0, 0)])
def test_multiquery_slots_padding_and_protection(kv4, S, R):
    """Qwen shapes (the multi-column kernel) with permuted side-cache slots,
    spare pages in the pool, page tables wider than needed, and protection
    widths that end inside a page."""
    from harness import build_from_host

    lengths = np.array([0, 1, 15, 16, 17, 143, 144, 145, 700, 1300], dtype=np.int32)
    wl = build_from_host(1, 0, lengths=lengths, n_sink=S, n_recent=R, slot_perm_seed=5, extra_pages=7,
                         max_pages=100)
    _check(kv4, wl, 6, f"qwen shapes S={S} R={R} permuted slots")


def test_multiquery_rejects_bad_counts(kv4):
    import torch

    from harness import build_from_host

    wl = build_from_host(0, 0, lengths=np.array([40, 50], dtype=np.int32))
    cfg = get_config(0)
    q = torch.zeros((2, 1, cfg.num_q_heads, cfg.head_dim), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros_like(q)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    for bad in (0, -1, kv4.MAX_QUERIES + 1):
        with pytest.raises(kv4.Kv4Error):
            kv4.decode_mq(wl.cache, wl.batch, q, bad, out, None, ws)
    # a workspace sized for one query per sequence is too small for eight
    T = 8
    q8 = torch.zeros((2, T, cfg.num_q_heads, cfg.head_dim), dtype=torch.bfloat16, device="cuda")
    small = torch.empty(kv4.workspace_bytes(wl.layout, 2, wl.alloc.page_table.shape[1]), dtype=torch.uint8,
                        device="cuda")
    with pytest.raises(kv4.Kv4Error):
        kv4.decode_mq(wl.cache, wl.batch, q8, T, torch.zeros_like(q8), None, small)


def test_multiquery_t64_qwen_shapes(kv4):
    """The largest query count (KV4_MAX_QUERIES = 64) at Hq 32 / Hkv 8 / D 128:
    16 blocks of four queries per sequence in the multi-column kernel, split
    sequences, and sequences shorter than T."""
    from harness import build_from_host

    assert kv4.MAX_QUERIES == 64
    lengths = np.array([2100, 300, 64, 40, 700, 145, 1], dtype=np.int32)
    wl = build_from_host(1, 0, lengths=lengths)
    _check(kv4, wl, 64, "qwen shapes T=64")


@pytest.mark.parametrize("fmt", [0, 1], ids=["kv4", "kv8"])
def test_chunked_prefill_256_in_4x64(kv4, fmt):
    """A 256-token prompt built as four chunks of 64 tokens: after each chunk
    is appended, one multi-query call attends its 64 positions causally over
    the cache as it stands (query t of the chunk sees everything before it
    and itself).  Qwen shapes with 16 sinks + 128 recent, so the middle INT4
    region first appears in the third chunk.  Each chunk's cache bytes and
    outputs are checked against the oracle given the same chunks.  kv4 runs
    the multi-column kernel; kv8 runs one single-query unit per query."""
    import torch

    from harness.device import _bf16, _i32
    from workloads import host_sequence

    cfg = get_config(1)
    B, P, T = 6, 256, 64
    S, R = (cfg.n_sink, cfg.n_recent) if fmt == 0 else (0, 0)
    lay = kv4.make_layout(cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, S, R)
    olay = oracle.make_layout(cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, S, R)
    npg = P // 16
    # pages of sequence b are b*npg .. b*npg + npg - 1 in both caches, so the
    # pools can be compared byte for byte
    pt = np.arange(B * npg, dtype=np.int32).reshape(B, npg)
    cache = kv4.alloc_cache(fmt, lay, B * npg, B)
    ocache = oracle.HostCache(fmt, olay, B * npg, B)
    toks = [host_sequence(cfg, 0, b, P)[:2] for b in range(B)]
    ws = torch.empty(kv4.workspace_bytes(lay, B * T, npg), dtype=torch.uint8, device="cuda")
    cu = np.arange(B + 1, dtype=np.int32) * T
    for c in range(P // T):
        n = (c + 1) * T
        lens = np.full(B, n, dtype=np.int32)
        k = np.concatenate([toks[b][0][c * T:n] for b in range(B)])
        v = np.concatenate([toks[b][1][c * T:n] for b in range(B)])
        batch = kv4.Batch(_i32(pt, "cuda"), _i32(lens, "cuda"))
        kv4.append(cache, batch, _bf16(k, "cuda"), _bf16(v, "cuda"), _i32(cu, "cuda"))
        oracle.append(ocache, pt, lens, None, k, v, cu)
        qh = host_queries(cfg, 10 + c, B, T)
        q = torch.from_numpy(qh.view(np.int16)).to("cuda").view(torch.bfloat16)
        out = torch.zeros((B, T, cfg.num_q_heads, cfg.head_dim), dtype=torch.bfloat16, device="cuda")
        lse = torch.zeros((B, T, cfg.num_q_heads), dtype=torch.float32, device="cuda")
        kv4.decode_mq(cache, batch, q, T, out, lse, ws)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(cache.pages.cpu().numpy(), ocache.pages, err_msg=f"chunk {c}: pages")
        if cache.side is not None:
            np.testing.assert_array_equal(cache.side.cpu().numpy(), ocache.side[:cache.side.numel()],
                                          err_msg=f"chunk {c}: side cache")
        out64, lse64, gap = oracle.decode_mq(ocache, pt, lens, None, qh, T)
        og = pu.bf16_bits_to_f64(out.view(torch.int16).cpu().numpy())
        m = pu.metrics_from(og, lse.cpu().numpy().astype(np.float64), out64, lse64, gap)
        print(f"\nprefill fmt={fmt} chunk {c} (positions {c * T}..{n - 1}): rel_l2={m['rel_l2']:.3e} "
              f"max_abs={m['max_abs']:.3e} lse={m['lse_abs']:.3e}", flush=True)
        pu.assert_within(m)
