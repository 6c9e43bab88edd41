"""Pins for the oracle's block layout, regions and side-cache rows.

The pages fix only "paged INT4" plus an INT8 side cache bounded at 144
positions for sinks and recent context (news summary "Async RL squeezes
context into fewer decode steps; ...", Interpretation paragraph 3).  The
layout is this implementation's; what is pinned here is that it is a
bijection (append then gather returns the exact values when the inputs are
exactly representable), the closed-form sizes, and the region algebra.
"""
import numpy as np
import pytest

from workloads import bf16_bits_from_f32


def exact_int4_rows(rng, n, H, D):
    """Rows whose 32-channel groups are integers in [-7, 7] times 2^e with a
    +-7 in every group, so INT4 quantization is exact."""
    codes = rng.integers(-7, 8, size=(n, H, D))
    codes[:, :, ::32] = 7 * rng.choice([-1, 1], size=(n, H, D // 32))
    e = rng.integers(-6, 6, size=(n, H, D // 32))
    x = codes.astype(np.float32) * np.repeat(np.float32(2.0) ** e, 32, axis=2)
    return bf16_bits_from_f32(x), x.astype(np.float64)


def exact_int8_rows(rng, n, H, D):
    codes = rng.integers(-127, 128, size=(n, H, D))
    codes[:, :, 0] = 127 * rng.choice([-1, 1], size=(n, H))
    e = rng.integers(-6, 6, size=(n, H, 1))
    x = codes.astype(np.float32) * (np.float32(2.0) ** e)
    return bf16_bits_from_f32(x), x.astype(np.float64)


def test_block_sizes_closed_form(orc):
    for D in (64, 128):
        lay = orc.make_layout(8, 8, D, 16, 128)
        assert orc.block_bytes(orc.FMT_KV4, lay) == 16 * D // 2 * 2 + 2 * 2 * (D // 32) * 16
        assert orc.block_bytes(orc.FMT_KV8, lay) == 16 * (2 * D + 4)
        assert orc.block_bytes(orc.FMT_BF16, lay) == 16 * 4 * D
    # S + R = 144 at D = 128: 144 rows of 2*128 code bytes + 2*2 scale bytes
    assert orc.side_bytes(orc.make_layout(32, 8, 128, 16, 128)) == 37440
    assert orc.side_bytes(orc.make_layout(4, 2, 64, 4, 16)) == 2 * 16 * (2 * 64 + 4)
    assert orc.side_bytes(orc.make_layout(4, 2, 64, 0, 0)) == 0


@pytest.mark.parametrize("S,R", [(4, 16), (16, 128), (0, 0), (0, 16), (4, 0), (144, 0), (0, 144), (5, 7)])
def test_region_algebra_exhaustive(orc, S, R):
    for n in range(0, 301):
        se, mb, me, rb = orc.regions(n, S, R)
        reg = np.full(n, -1)
        reg[:se] = 0
        reg[mb:me] = 1
        assert np.all(reg[rb:n] == -1) or rb == n
        reg[rb:n] = 2
        assert np.all(reg >= 0), "every position is in a region"
        counts = [(reg == r).sum() for r in range(3)]
        assert counts[0] + counts[1] + counts[2] == n
        assert counts[0] == min(S, n)
        assert counts[0] + counts[2] == min(n, S + R), "protected = min(n, S+R)"
        assert counts[2] <= R
        # sinks are the first positions, recent the last, middle contiguous
        if counts[2]:
            assert rb == n - counts[2] and rb >= S
        if counts[1]:
            assert mb == S and me == n - R
        # side rows of the protected positions are distinct and inside the side block
        rows = [orc.side_row(p, S, R) for p in range(n) if reg[p] != 1]
        assert len(set(rows)) == len(rows)
        assert all(0 <= r < S + R for r in rows)


@pytest.mark.parametrize("fmt,D", [(0, 64), (0, 128), (1, 64), (1, 128), (2, 64), (2, 128)])
def test_append_gather_roundtrip_exact(orc, fmt, D):
    """Exactly representable rows come back unchanged from every position."""
    rng = np.random.default_rng(3 + fmt + D)
    H, n = 2, 70
    S, R = (4, 16) if fmt == orc.FMT_KV4 else (0, 0)
    lay = orc.make_layout(2 * H, H, D, S, R)
    if fmt == orc.FMT_KV8:
        kb, kx = exact_int8_rows(rng, n, H, D)
        vb, vx = exact_int8_rows(rng, n, H, D)
    elif fmt == orc.FMT_KV4:
        # middle positions exact in INT4, protected positions exact in INT8
        kb, kx = exact_int4_rows(rng, n, H, D)
        vb, vx = exact_int4_rows(rng, n, H, D)
        prot = np.r_[0:S, n - R:n]
        kb[prot], kx[prot] = exact_int8_rows(rng, prot.size, H, D)
        vb[prot], vx[prot] = exact_int8_rows(rng, prot.size, H, D)
    else:
        kx = rng.standard_normal((n, H, D)).astype(np.float32)
        vx = rng.standard_normal((n, H, D)).astype(np.float32)
        kb, vb = bf16_bits_from_f32(kx), bf16_bits_from_f32(vx)
        kx = kb.astype(np.uint32).__lshift__(16).view(np.float32).astype(np.float64)
        vx = vb.astype(np.uint32).__lshift__(16).view(np.float32).astype(np.float64)
    npages = (n + 15) // 16
    pt = rng.permutation(npages + 3)[:npages].astype(np.int32)[None, :]
    cache = orc.HostCache(fmt, lay, num_pages=npages + 3, num_slots=1)
    orc.append(cache, pt, np.array([n], np.int32), None, kb, vb, np.array([0, n], np.int32))
    for h in range(H):
        K, V, reg = orc.gather(cache, pt, np.array([n], np.int32), None, 0, h)
        if fmt == orc.FMT_KV4:
            # the INT4 exact rows are also INT8 exact, so protected rows match too
            assert reg[:S].tolist() == [0] * S and reg[n - R:].tolist() == [2] * R
        np.testing.assert_array_equal(K, kx[:, h, :])
        np.testing.assert_array_equal(V, vx[:, h, :])


@pytest.mark.parametrize("fmt,D", [(0, 64), (0, 128), (1, 128), (2, 64)])
def test_code_area_is_a_bijection(orc, fmt, D):
    """A full page of distinct (row, channel) codes covers every code byte once."""
    lay = orc.make_layout(1, 1, D, 0, 0)
    rng = np.random.default_rng(99)
    if fmt == orc.FMT_KV4:
        kb, _ = exact_int4_rows(rng, 16, 1, D)
    elif fmt == orc.FMT_KV8:
        kb, _ = exact_int8_rows(rng, 16, 1, D)
    else:
        kb = bf16_bits_from_f32(rng.standard_normal((16, 1, D)).astype(np.float32))
    cache = orc.HostCache(fmt, lay, num_pages=1, num_slots=1)
    cache.pages[:] = 0xA5  # poison: every code byte must be overwritten
    orc.append(cache, np.zeros((1, 1), np.int32), np.array([16], np.int32), None, kb, kb,
               np.array([0, 16], np.int32))
    bb = orc.block_bytes(fmt, lay)
    # K and V code areas hold the same multiset of codes (same input rows)
    if fmt == orc.FMT_KV4:
        karea, varea = cache.pages[:8 * D], cache.pages[8 * D:16 * D]
        nib = lambda a: np.sort(np.concatenate([a & 15, a >> 4]))
        np.testing.assert_array_equal(nib(karea), nib(varea))
    elif fmt == orc.FMT_KV8:
        np.testing.assert_array_equal(np.sort(cache.pages[:16 * D]), np.sort(cache.pages[16 * D:32 * D]))
    else:
        k16 = cache.pages[:32 * D].view(np.uint16)
        v16 = cache.pages[32 * D:64 * D].view(np.uint16)
        np.testing.assert_array_equal(np.sort(k16), np.sort(v16))
        np.testing.assert_array_equal(np.sort(k16), np.sort(kb.ravel()))
    # nothing outside the block was touched
    assert cache.pages.size == bb


def test_sink_and_ring_hold_the_right_positions(orc):
    """Token-by-token appends: sinks keep positions 0..S-1, the ring the last R."""
    rng = np.random.default_rng(21)
    D, H, S, R = 64, 1, 4, 16
    lay = orc.make_layout(1, H, D, S, R)
    n_total = 57
    kb, kx = exact_int8_rows(rng, n_total, H, D)
    vb, vx = exact_int8_rows(rng, n_total, H, D)
    npages = (n_total + 15) // 16
    pt = np.arange(npages, dtype=np.int32)[None, :]
    cache = orc.HostCache(orc.FMT_KV4, lay, num_pages=npages, num_slots=1)
    for n in range(1, n_total + 1):
        orc.append(cache, pt, np.array([n], np.int32), None, kb[n - 1:n], vb[n - 1:n],
                   np.array([0, 1], np.int32))
        K, V, reg = orc.gather(cache, pt, np.array([n], np.int32), None, 0, 0)
        prot = reg != 1
        # INT8-exact rows come back exactly from the side cache at protected positions
        np.testing.assert_array_equal(K[prot], kx[:n, 0][prot])
        np.testing.assert_array_equal(V[prot], vx[:n, 0][prot])
        assert prot.sum() == min(n, S + R)
