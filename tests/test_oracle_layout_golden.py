"""Pins for the cache byte layout: hand-worked byte offsets and nibbles.

The pages fix only "paged INT4" plus an INT8 side cache for sinks and recent
positions (news summary "Async RL squeezes context into fewer decode steps;
...", Interpretation paragraph 3); the block layout is this library's and is
stated in include/kv4.h.  tests/golden/layout_cases.txt works out, by hand,
where single codes and scales land for K and V of INT4 pages, INT8 pages, the
INT8 side tile and bf16 pages.  A swapped nibble, a transposed (position,
channel) index or a wrong word order in the oracle's writer moves a byte and
fails these cases.
"""
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "layout_cases.txt")
FORMATS = {"kv4": 0, "kv8": 1, "bf16": 2}


def _cases():
    out = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            cid, fmt, D, prot, area, inputs, want = [p.strip() for p in line.split("|")]
            S, R = (int(v) for v in prot.split(","))
            vals = []
            for item in inputs.split(";"):
                which, r, c, bits = item.split()
                vals.append((which, int(r), int(c), int(bits, 16)))
            expect = {}
            for item in want.split():
                off, byte = item.split(":")
                expect[int(off)] = int(byte, 16)
            out.append(dict(id=cid, fmt=FORMATS[fmt], D=int(D), S=S, R=R, area=area, vals=vals,
                            expect=expect))
    return out


CASES = _cases()


def case_inputs(c):
    """bf16 bit arrays K, V [16][1][D] of the case (one page, one kv head)."""
    D = c["D"]
    k = np.zeros((16, 1, D), dtype=np.uint16)
    v = np.zeros((16, 1, D), dtype=np.uint16)
    for which, r, ch, bits in c["vals"]:
        (k if which == "K" else v)[r, 0, ch] = bits
    return k, v


def expected_buffer(c, size):
    want = np.zeros(size, dtype=np.uint8)
    for off, byte in c["expect"].items():
        want[off] = byte
    return want


@pytest.mark.parametrize("c", CASES, ids=[c["id"] for c in CASES])
def test_layout_case_oracle(orc, c):
    lay = orc.make_layout(1, 1, c["D"], c["S"], c["R"])
    cache = orc.HostCache(c["fmt"], lay, num_pages=1, num_slots=1)
    k, v = case_inputs(c)
    orc.append(cache, np.zeros((1, 1), np.int32), np.array([16], np.int32), None, k, v,
               np.array([0, 16], np.int32))
    if c["area"] == "page":
        got = cache.pages
        assert got.size == orc.block_bytes(c["fmt"], lay)
    else:
        got = cache.side[:orc.side_bytes(lay)]
    want = expected_buffer(c, got.size)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{c['id']}: bytes differ at {bad[:8].tolist()}: got {got[bad[:8]].tolist()}"
