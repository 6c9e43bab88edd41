"""Pins for the oracle's multi-query decode.

The pages describe the single-token decode step over the INT4 cache with INT8
sink and recent copies (news summary "Async RL squeezes context into fewer
decode steps; ...", Interpretation paragraph 3).  Running T query tokens over
one cache state is a reading of this library: query t sits at position
N - T + t and sees the first N - T + t + 1 positions, each read from where
the cache holds it after the append.  The pins tie that reading to things
computed another way: torch's scaled_dot_product_attention in float64 with an
explicit causal mask over the full gathered rows, the single-token decode
(T = 1, the last query, and the unprotected cache where no position depends
on the cache state), and the empty queries of T > N.
"""
import numpy as np
import pytest

from workloads import f32_from_bf16_bits, get_config, host_queries, host_sequence

from test_oracle_attention import build_host_cache


def _q_single(q_mq, t):
    """The [B][Hq][D] slice of query t."""
    return np.ascontiguousarray(q_mq[:, t])


@pytest.mark.parametrize("S,R,T", [(4, 16, 1), (4, 16, 5), (4, 4, 9), (0, 0, 6), (16, 8, 3)])
def test_multiquery_vs_masked_sdpa(orc, S, R, T):
    """Every query against torch SDPA (float64) over all N gathered rows with a
    boolean mask that keeps positions [0, N - T + t + 1)."""
    torch = pytest.importorskip("torch")
    cfg = get_config(0)
    lengths = np.array([70, 33, 6, 19], dtype=np.int32)
    cache, alloc, _ = build_host_cache(orc, cfg, orc.FMT_KV4, lengths, S=S, R=R)
    q = host_queries(cfg, 0, lengths.size, T)
    out, lse, gap = orc.decode_mq(cache, alloc.page_table, lengths, None, q, T)
    assert gap <= 1e-12
    g = cfg.g
    for b, N in enumerate(lengths):
        for h in range(cfg.num_kv_heads):
            K, V, _ = orc.gather(cache, alloc.page_table, lengths, None, b, h)
            for t in range(T):
                n = int(N) - T + t + 1
                qh = f32_from_bf16_bits(q[b, t, h * g:(h + 1) * g]).astype(np.float64)
                if n <= 0:
                    assert np.all(out[b, t, h * g:(h + 1) * g] == 0.0)
                    assert np.all(np.isneginf(lse[b, t, h * g:(h + 1) * g]))
                    continue
                tq = torch.from_numpy(qh)[None, :, None, :]
                tk = torch.from_numpy(K)[None, None].expand(1, g, -1, -1).contiguous()
                tv = torch.from_numpy(V)[None, None].expand(1, g, -1, -1).contiguous()
                mask = torch.zeros((1, 1, 1, K.shape[0]), dtype=torch.bool)
                mask[..., :n] = True
                ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask,
                                                                       scale=1.0)
                np.testing.assert_allclose(out[b, t, h * g:(h + 1) * g], ref[0, :, 0].numpy(),
                                           rtol=1e-10, atol=1e-12)
                s = qh @ K[:n].T
                m = s.max(axis=1, keepdims=True)
                np.testing.assert_allclose(lse[b, t, h * g:(h + 1) * g],
                                           (m + np.log(np.exp(s - m).sum(axis=1, keepdims=True)))[:, 0],
                                           rtol=1e-12)


def test_single_query_and_last_query_equal_decode(orc):
    """T = 1 is the single-token decode; for any T the last query sees the
    whole cache and equals the single-token decode with its q."""
    cfg = get_config(0)
    lengths = np.array([300, 57, 17, 3], dtype=np.int32)
    cache, alloc, _ = build_host_cache(orc, cfg, orc.FMT_KV4, lengths)
    for T in (1, 4):
        q = host_queries(cfg, 0, lengths.size, T)
        out, lse, _ = orc.decode_mq(cache, alloc.page_table, lengths, None, q, T)
        o1, l1, _ = orc.decode(cache, alloc.page_table, lengths, None, _q_single(q, T - 1))
        np.testing.assert_array_equal(out[:, T - 1], o1)
        np.testing.assert_array_equal(lse[:, T - 1], l1)


def test_integer_query_last_query_equals_decode(orc):
    """With the integer-query variant the last query still equals the
    single-token decode with the same variant, and the variant differs from
    the bf16 query."""
    cfg = get_config(0)
    lengths = np.array([300, 57, 17], dtype=np.int32)
    cache, alloc, _ = build_host_cache(orc, cfg, orc.FMT_KV4, lengths)
    T = 3
    q = host_queries(cfg, 0, lengths.size, T)
    out, lse, _ = orc.decode_mq(cache, alloc.page_table, lengths, None, q, T, q_int8=True)
    o1, l1, _ = orc.decode(cache, alloc.page_table, lengths, None, _q_single(q, T - 1), q_int8=True)
    np.testing.assert_array_equal(out[:, T - 1], o1)
    np.testing.assert_array_equal(lse[:, T - 1], l1)
    outf, _, _ = orc.decode_mq(cache, alloc.page_table, lengths, None, q, T)
    assert not np.array_equal(out, outf)


@pytest.mark.parametrize("fmt", [0, 1, 2], ids=["kv4-plain", "kv8", "bf16"])
def test_unprotected_query_equals_decode_of_prefix(orc, fmt):
    """Without a side cache no row depends on the cache state, so query t
    equals the single-token decode of the same cache at length N - T + t + 1
    (region bookkeeping of its own)."""
    cfg = get_config(0)
    lengths = np.array([90, 41, 8], dtype=np.int32)
    cache, alloc, _ = build_host_cache(orc, cfg, fmt, lengths, S=0, R=0)
    T = 6
    q = host_queries(cfg, 0, lengths.size, T)
    out, lse, _ = orc.decode_mq(cache, alloc.page_table, lengths, None, q, T)
    for t in range(T):
        n = np.maximum(lengths - T + t + 1, 0).astype(np.int32)
        o1, l1, _ = orc.decode(cache, alloc.page_table, n, None, _q_single(q, t))
        np.testing.assert_allclose(out[:, t], o1, rtol=0, atol=1e-15)
        np.testing.assert_array_equal(np.isneginf(lse[:, t]), np.isneginf(l1))
        fin = np.isfinite(l1)
        np.testing.assert_allclose(lse[:, t][fin], l1[fin], rtol=0, atol=1e-15)


def _cache_of_prefix(orc, cfg, k, v, n, S, R):
    """Oracle cache holding the first n of the given tokens (one sequence)."""
    lay = orc.make_layout(cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, S, R)
    npg = max(1, (n + 15) // 16)
    pt = np.arange(npg, dtype=np.int32)[None, :]
    cache = orc.HostCache(orc.FMT_KV4, lay, npg, 1)
    orc.append(cache, pt, np.array([n], np.int32), None, k[:n], v[:n], np.array([0, n], np.int32))
    return cache, pt


def test_protected_rows_follow_the_cache_state(orc):
    """With protection, a query that ends before the ring reads INT4 for
    positions a shorter cache would have held in INT8: its output differs from
    the decode of the same tokens' shorter cache exactly when such positions
    exist."""
    cfg = get_config(0)
    N, S, R, T = 64, 4, 16, 12
    k, v, _ = host_sequence(cfg, 0, 0, N)
    full, pt = _cache_of_prefix(orc, cfg, k, v, N, S, R)
    q = host_queries(cfg, 0, 1, T)
    out, _, _ = orc.decode_mq(full, pt, np.array([N], np.int32), None, q, T)
    ring0 = max(S, N - R)
    outcomes = []
    for t in range(T):
        n = N - T + t + 1
        # a cache of n positions holds [max(S, n - R), n) in INT8; the full
        # one holds only [ring0, n) there
        mismatch = max(S, n - R) < ring0
        short, spt = _cache_of_prefix(orc, cfg, k, v, n, S, R)
        o1, _, _ = orc.decode(short, spt, np.array([n], np.int32), None, _q_single(q, t))
        same = np.array_equal(out[:, t], o1)
        outcomes.append((mismatch, same))
        assert same != mismatch, (t, n)
    assert any(m for m, _ in outcomes) and any(not m for m, _ in outcomes)
