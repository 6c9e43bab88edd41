"""Pins for the capacity model (host arithmetic; no GPU).

The pages credit part of the end-to-end gain to the higher concurrency a
smaller cache allows, and note that a fixed page budget limits the scheduling
benefit (news summary "Async RL squeezes context into fewer decode steps;
...", Perspective paragraphs 1 and 2).  The model counts whole pages per
sequence and layer, plus the fixed INT8 side block of KV4 with protection.
The oracle is pinned to closed forms typed from the block layout and to
brute-force prefix sums; the library's host function must equal the oracle.
"""
import math

import numpy as np
import pytest

from workloads import get_config, context_lengths


def _closed_form(fmt, D, Hkv, S, R, layers, lengths):
    block = {0: 18 * D, 1: 32 * D + 64, 2: 64 * D}[fmt]
    pages = sum(math.ceil(int(n) / 16) for n in lengths)
    side = 0
    if fmt == 0 and S + R > 0:
        side = len(lengths) * math.ceil((S + R) / 16) * (32 * D + 64)
    return layers * Hkv * (pages * block + side)


@pytest.mark.parametrize("fmt", [0, 1, 2])
@pytest.mark.parametrize("S,R", [(16, 128), (0, 0), (4, 16)])
def test_oracle_capacity_closed_form_and_prefix_fit(orc, fmt, S, R):
    rng = np.random.default_rng(7)
    lengths = rng.integers(0, 5000, size=57).astype(np.int32)
    lengths[3] = 0
    lengths[5] = 16
    lengths[6] = 17
    lay = orc.make_layout(32, 8, 128, S, R)
    total, fit = orc.cache_capacity(fmt, lay, 36, lengths, 0)
    assert total == _closed_form(fmt, 128, 8, S, R, 36, lengths)
    # a budget below the first sequence fits none (the side block alone is
    # nonzero with protection; a length-0 sequence without it fits anywhere)
    per = [_closed_form(fmt, 128, 8, S, R, 36, [n]) for n in lengths]
    cums = np.cumsum(per)
    for budget in (0, int(cums[10]), int(cums[10]) - 1, int(cums[-1]), int(cums[-1]) + 12345, int(cums[30]) + 1):
        _, f = orc.cache_capacity(fmt, lay, 36, lengths, budget)
        want = int(np.searchsorted(cums, budget, side="right"))
        assert f == want, (budget, f, want)


def test_format_ratios_for_long_contexts(orc):
    """Per position and kv head: BF16 512 B, INT8 260 B, INT4 144 B; the
    protected side block is fixed per sequence, so its share vanishes with
    length."""
    lay = orc.make_layout(32, 8, 128, 16, 128)
    lengths = np.full(64, 16 * 4096, dtype=np.int32)
    b = {f: orc.cache_capacity(f, lay, 1, lengths, 0)[0] for f in (0, 1, 2)}
    assert b[2] / b[1] == pytest.approx(512 / 260, rel=1e-12)
    # the side block (9 x 4160 B per kv head) is 0.4% of a 64k-position sequence
    assert b[2] / b[0] == pytest.approx(512 / (144 + 9 * 4160 / (16 * 4096)), rel=1e-12)
    lay0 = orc.make_layout(32, 8, 128, 0, 0)
    plain = orc.cache_capacity(0, lay0, 1, lengths, 0)[0]
    assert b[2] / plain == pytest.approx(512 / 144, rel=1e-12)
    assert b[0] - plain == 64 * 8 * 9 * (32 * 128 + 64)


def test_library_capacity_equals_oracle(orc):
    """The C-ABI host function (no device call) against the oracle, on the
    config-2 length distribution, every format and several budgets."""
    import int4_kv_cache_amd as kv4

    kv4.load()
    cfg = get_config(2)
    lengths = context_lengths(cfg)
    for fmt in (0, 1, 2):
        S, R = (16, 128) if fmt == 0 else (0, 0)
        lay = kv4.make_layout(cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, S, R)
        olay = orc.make_layout(cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, S, R)
        for budget in (0, 10**9, 240 * 10**9, 10**15):
            assert kv4.cache_capacity(lay, fmt, 36, lengths, budget) == \
                orc.cache_capacity(fmt, olay, 36, lengths, budget)


def test_library_capacity_rejects_bad_input():
    import int4_kv_cache_amd as kv4

    kv4.load()
    lay = kv4.make_layout(32, 8, 128, 16, 128)
    with pytest.raises(kv4.Kv4Error):
        kv4.cache_capacity(lay, 0, 36, np.array([5, -1], np.int32), 10**9)
    with pytest.raises(kv4.Kv4Error):
        kv4.cache_capacity(lay, 3, 36, np.array([5], np.int32), 10**9)
    with pytest.raises(kv4.Kv4Error):
        kv4.cache_capacity(lay, 0, 0, np.array([5], np.int32), 10**9)
    assert kv4.cache_capacity(lay, 0, 36, np.zeros(0, np.int32), 10**9) == (0, 0)
