"""Pins for the oracle's attention, regional merge and decode.

The method evaluates attention region by region (INT8 sinks, INT4 middle,
INT8 recent) and combines the regions by an exact softmax merge (news
summary "Async RL squeezes context into fewer decode steps; ...",
Interpretation paragraph 3).  Exact means the merge equals one softmax over
all positions; the pins are that identity, brute force with math.fsum and no
max-shift, torch's scaled_dot_product_attention in float64 on the CPU, and
closed-form special cases.
"""
import math

import numpy as np
import pytest

from workloads import bf16_bits_from_f32, f32_from_bf16_bits, get_config, host_sequence, PageAllocator


def brute_attention(q, K, V):
    """softmax(q.K^T) V with exp(s) / fsum(exp(s)) -- no max shift."""
    n, D = K.shape
    s = [math.fsum(float(q[c]) * float(K[j, c]) for c in range(D)) for j in range(n)]
    e = [math.exp(x) for x in s]
    tot = math.fsum(e)
    out = [math.fsum(e[j] * float(V[j, c]) for j in range(n)) / tot for c in range(D)]
    return np.array(out), math.log(tot)


@pytest.mark.parametrize("seed", range(12))
def test_attend_vs_brute_force(orc, seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 41))
    D = int(rng.choice([2, 4, 8]))
    q = rng.standard_normal(D)
    K = rng.standard_normal((n, D)) * 1.5
    V = rng.standard_normal((n, D))
    region = np.sort(rng.integers(0, 3, size=n)).astype(np.uint8)
    out, lse, gap = orc.attend(q, K, V, region)
    want, wlse = brute_attention(q, K, V)
    np.testing.assert_allclose(out, want, rtol=1e-12, atol=1e-13)
    assert abs(lse - wlse) <= 1e-12 * max(1.0, abs(wlse))
    assert gap <= 1e-12


def test_merge_identity_large_scores(orc):
    """Regions whose maxima differ by hundreds still merge exactly."""
    rng = np.random.default_rng(1)
    n, D = 300, 16
    q = rng.standard_normal(D)
    K = rng.standard_normal((n, D)) * 40
    V = rng.standard_normal((n, D))
    region = np.array([0] * 10 + [1] * 250 + [2] * 40, dtype=np.uint8)
    out, lse, gap = orc.attend(q, K, V, region)
    assert gap <= 1e-12
    s = K @ q
    m = s.max()
    w = np.exp(s - m)
    np.testing.assert_allclose(out, (w @ V) / w.sum(), rtol=1e-11, atol=1e-12)
    assert abs(lse - (m + math.log(w.sum()))) < 1e-10


def test_special_cases(orc):
    rng = np.random.default_rng(2)
    D = 16
    V = rng.standard_normal((9, D))
    K = rng.standard_normal((9, D))
    # one position: the output is that value row, lse is its score
    out, lse, _ = orc.attend(rng.standard_normal(D), K[:1], V[:1], None, 0.5)
    np.testing.assert_array_equal(out, V[0])
    # q = 0: uniform weights, output is the mean of V, lse = ln n
    out, lse, _ = orc.attend(np.zeros(D), K, V)
    np.testing.assert_allclose(out, V.mean(axis=0), rtol=1e-13, atol=1e-14)
    assert abs(lse - math.log(9)) < 1e-14
    # all keys equal: uniform again
    Ke = np.repeat(K[:1], 9, axis=0)
    out, _, _ = orc.attend(rng.standard_normal(D), Ke, V)
    np.testing.assert_allclose(out, V.mean(axis=0), rtol=1e-13, atol=1e-14)
    # empty context: zeros and lse = -inf
    out, lse, _ = orc.attend(rng.standard_normal(D), np.zeros((0, D)), np.zeros((0, D)))
    assert np.all(out == 0) and lse == -math.inf
    # the softmax scale multiplies q.k
    q = rng.standard_normal(D)
    a, la, _ = orc.attend(q, K, V, None, 0.25)
    b, lb, _ = orc.attend(q * 0.25, K, V, None, 1.0)
    np.testing.assert_allclose(a, b, rtol=1e-14, atol=1e-15)


def build_host_cache(orc, cfg, fmt, lengths, S=None, R=None, perm_seed=0, token_by_token=False):
    """Append every sequence of a small workload through the oracle."""
    S = cfg.n_sink if S is None else S
    R = cfg.n_recent if R is None else R
    lay = orc.make_layout(cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, S, R)
    alloc = PageAllocator(lengths, seed=perm_seed)
    cache = orc.HostCache(fmt, lay, alloc.num_pages, len(lengths))
    qs = []
    for b, n in enumerate(lengths):
        k, v, q = host_sequence(cfg, 0, b, int(n))
        qs.append(q)
        sl = np.zeros(len(lengths), np.int32)
        if token_by_token:
            for p in range(int(n)):
                sl[b] = p + 1
                cu = np.zeros(len(lengths) + 1, np.int32)
                cu[b + 1:] = 1
                orc.append(cache, alloc.page_table, sl, None, k[p:p + 1], v[p:p + 1], cu)
        else:
            sl[b] = n
            cu = np.zeros(len(lengths) + 1, np.int32)
            cu[b + 1:] = n
            orc.append(cache, alloc.page_table, sl, None, k, v, cu)
    return cache, alloc, np.stack(qs)


def test_bulk_and_token_by_token_append_identical(orc):
    """Calibration-free: the bytes do not depend on how tokens arrive."""
    cfg = get_config(0)
    lengths = [37, 70]
    a, _, _ = build_host_cache(orc, cfg, orc.FMT_KV4, lengths)
    b, _, _ = build_host_cache(orc, cfg, orc.FMT_KV4, lengths, token_by_token=True)
    np.testing.assert_array_equal(a.pages, b.pages)
    # side blocks: only the rows holding live positions are defined
    np.testing.assert_array_equal(a.side, b.side)


def test_decode_vs_torch_sdpa_and_page_permutation(orc):
    torch = pytest.importorskip("torch")
    cfg = get_config(0)
    lengths = np.array([300, 517, 5, 21], dtype=np.int32)
    cache, alloc, q = build_host_cache(orc, cfg, orc.FMT_KV4, lengths)
    out, lse, gap = orc.decode(cache, alloc.page_table, lengths, None, q)
    assert gap <= 1e-12
    g = cfg.g
    for b in range(lengths.size):
        for h in range(cfg.num_kv_heads):
            K, V, _ = orc.gather(cache, alloc.page_table, lengths, None, b, h)
            qh = f32_from_bf16_bits(q[b, h * g:(h + 1) * g]).astype(np.float64)
            tq = torch.from_numpy(qh)[None, :, None, :]            # [1, g, 1, D]
            tk = torch.from_numpy(K)[None, None].expand(1, g, -1, -1).contiguous()
            tv = torch.from_numpy(V)[None, None].expand(1, g, -1, -1).contiguous()
            ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=1.0)
            np.testing.assert_allclose(out[b, h * g:(h + 1) * g], ref[0, :, 0].numpy(),
                                       rtol=1e-10, atol=1e-12)
            s = qh @ K.T
            m = s.max(axis=1, keepdims=True)
            np.testing.assert_allclose(lse[b, h * g:(h + 1) * g],
                                       (m + np.log(np.exp(s - m).sum(axis=1, keepdims=True)))[:, 0],
                                       rtol=1e-12)
    # a different physical page assignment gives identical outputs
    cache2, alloc2, _ = build_host_cache(orc, cfg, orc.FMT_KV4, lengths, perm_seed=5)
    assert not np.array_equal(alloc.page_table, alloc2.page_table)
    out2, lse2, _ = orc.decode(cache2, alloc2.page_table, lengths, None, q)
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(lse, lse2)


def test_gqa_head_mapping(orc):
    """Query head hq reads kv head hq // g: swapping kv-head data swaps outputs."""
    cfg = get_config(0)
    lengths = np.array([40], dtype=np.int32)
    cache, alloc, q = build_host_cache(orc, cfg, orc.FMT_BF16, lengths)
    out, _, _ = orc.decode(cache, alloc.page_table, lengths, None, q)
    K0, V0, _ = orc.gather(cache, alloc.page_table, lengths, None, 0, 0)
    K1, V1, _ = orc.gather(cache, alloc.page_table, lengths, None, 0, 1)
    assert not np.allclose(K0, K1)
    for hq in range(cfg.num_q_heads):
        K, V = (K0, V0) if hq // cfg.g == 0 else (K1, V1)
        want, _ = brute_attention(f32_from_bf16_bits(q[0, hq]).astype(np.float64), K, V)
        np.testing.assert_allclose(out[0, hq], want, rtol=1e-11, atol=1e-12)


def test_variant_reductions(orc):
    """Closed-form relations between the cache formats.

    * context <= S + R: KV4-RL reads only INT8 copies -> equals all-INT8.
    * S = R = 0 with INT4-exact inputs: plain INT4 equals BF16.
    """
    cfg = get_config(0)
    short = np.array([20, 7, 1], dtype=np.int32)   # S + R = 20
    c4, a4, q = build_host_cache(orc, cfg, orc.FMT_KV4, short)
    c8, a8, _ = build_host_cache(orc, cfg, orc.FMT_KV8, short)
    o4, l4, _ = orc.decode(c4, a4.page_table, short, None, q)
    o8, l8, _ = orc.decode(c8, a8.page_table, short, None, q)
    np.testing.assert_allclose(o4, o8, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(l4, l8, rtol=1e-13)

    # INT4-exact data: integer codes times a power of two per 32-channel group
    rng = np.random.default_rng(8)
    D, H, n = 64, 2, 45
    codes = rng.integers(-7, 8, size=(n, H, D))
    codes[:, :, ::32] = 7
    x = codes.astype(np.float32) * np.float32(0.25)
    kb = bf16_bits_from_f32(x)
    vb = bf16_bits_from_f32(x[::-1].copy())
    qb = bf16_bits_from_f32(rng.standard_normal((1, 4, D)).astype(np.float32) * np.float32(0.1))
    outs = []
    for fmt, (S, R) in ((orc.FMT_KV4, (0, 0)), (orc.FMT_BF16, (0, 0))):
        lay = orc.make_layout(4, H, D, S, R)
        cache = orc.HostCache(fmt, lay, 3, 1)
        pt = np.array([[2, 0, 1]], np.int32)
        orc.append(cache, pt, np.array([n], np.int32), None, kb, vb, np.array([0, n], np.int32))
        outs.append(orc.decode(cache, pt, np.array([n], np.int32), None, qb)[0])
    np.testing.assert_allclose(outs[0], outs[1], rtol=1e-14, atol=1e-15)


def test_empty_sequence_decodes_to_zero(orc):
    cfg = get_config(0)
    lengths = np.array([0, 33], dtype=np.int32)
    cache, alloc, q = build_host_cache(orc, cfg, orc.FMT_KV4, lengths)
    out, lse, _ = orc.decode(cache, alloc.page_table, lengths, None, q)
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    assert np.all(np.isfinite(lse[1]))


def test_int8_query_exact_grid_equals_plain(orc):
    """A query already on the INT8 grid (integers times a power of two, largest
    |integer| 127) is reproduced exactly by the integer-query quantizer, so the
    integer-query decode equals the plain decode bit for bit."""
    cfg = get_config(0)
    lengths = np.array([300, 517], dtype=np.int32)
    cache, alloc, q = build_host_cache(orc, cfg, orc.FMT_KV4, lengths)
    rng = np.random.default_rng(9)
    ints = rng.integers(-127, 128, size=q.shape).astype(np.float32)
    ints[..., 0] = 127.0                                       # amax = 127 * 2^e in every row
    qx = bf16_bits_from_f32(ints * np.float32(2.0 ** -9))
    a = orc.decode(cache, alloc.page_table, lengths, None, qx)
    b = orc.decode(cache, alloc.page_table, lengths, None, qx, q_int8=True)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_int8_query_is_quantize_then_attend(orc):
    """The integer-query decode of head hq equals attention (oracle attend over
    the gathered rows) with that head's q replaced by its INT8 row codes x
    scale from the pinned quantizer -- checks which row is quantized for which
    head and sequence."""
    cfg = get_config(0)
    lengths = np.array([37, 300], dtype=np.int32)
    cache, alloc, q = build_host_cache(orc, cfg, orc.FMT_KV4, lengths)
    out, lse, _ = orc.decode(cache, alloc.page_table, lengths, None, q, q_int8=True)
    plain, _, _ = orc.decode(cache, alloc.page_table, lengths, None, q)
    assert np.abs(out - plain).max() > 0                       # the quantization does change q
    g = cfg.g
    for b in range(lengths.size):
        for h in range(cfg.num_kv_heads):
            K, V, reg = orc.gather(cache, alloc.page_table, lengths, None, b, h)
            for j in range(g):
                hq = h * g + j
                codes, sbits = orc.quant_sym(q[b, hq], 127)
                qv = codes.astype(np.float64) * orc.f16_to_f64(int(sbits))
                o, l, _ = orc.attend(qv, K, V, reg)
                np.testing.assert_array_equal(out[b, hq], o)
                assert lse[b, hq] == l
