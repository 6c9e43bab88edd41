"""Pins for the oracle's quantizer, fp16 rounding and nibble packing.

The quantizer follows the calibration-free INT4 rule (news summary "Async RL
squeezes context into fewer decode steps; ...", Synopsis) with the readings
listed in tests/golden/quantizer_cases.txt.  Pins: hand-worked cases (golden
file), numpy's float16 rounding (an independent library routine) and the
quantizer's invariants.
"""
import os

import numpy as np
import pytest

from workloads import bf16_bits_from_f32, f32_from_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quantizer_cases.txt")


def _cases():
    out = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            cid, qmax, n, xs, scale, codes, packed = [p.strip() for p in line.split("|")]
            out.append(dict(id=cid, qmax=int(qmax), n=int(n),
                            x=[int(v, 16) for v in xs.split()],
                            scale=int(scale, 16),
                            codes=[int(v) for v in codes.split()],
                            packed=[int(v, 16) for v in packed.split()]))
    return out


CASES = _cases()


def _full_input(c):
    x = np.zeros(c["n"], dtype=np.uint16)
    x[:len(c["x"])] = c["x"]
    return x


@pytest.mark.parametrize("c", CASES, ids=[c["id"] for c in CASES])
def test_hand_cases_codes_and_scale(orc, c):
    codes, scale = orc.quant_sym(_full_input(c), c["qmax"])
    assert scale == c["scale"]
    want = np.zeros(c["n"], dtype=np.int8)
    want[:len(c["codes"])] = c["codes"]
    np.testing.assert_array_equal(codes, want)


@pytest.mark.parametrize("c", CASES, ids=[c["id"] for c in CASES])
def test_hand_cases_packed_bytes(orc, c):
    """Append the case as row 0 of one page and read the K code bytes."""
    if c["qmax"] == 7:
        fmt, D = orc.FMT_KV4, 64          # two 32-channel groups, case in group 0
    else:
        fmt, D = orc.FMT_KV8, c["n"]
    lay = orc.make_layout(1, 1, D, 0, 0)
    cache = orc.HostCache(fmt, lay, num_pages=1, num_slots=1)
    k = np.zeros((1, 1, D), dtype=np.uint16)
    k[0, 0, :c["n"]] = _full_input(c)
    v = np.zeros_like(k)
    orc.append(cache, np.zeros((1, 1), np.int32), np.array([1], np.int32), None, k, v,
               np.array([0, 1], np.int32))
    got = cache.pages[:len(c["packed"])]
    np.testing.assert_array_equal(got, np.array(c["packed"], dtype=np.uint8))
    # the scale sits at the start of the K-scale area (group 0, row 0)
    off = 16 * D if fmt == orc.FMT_KV4 else 32 * D
    assert int(cache.pages[off]) | (int(cache.pages[off + 1]) << 8) == c["scale"]


def test_fp16_rounding_matches_numpy(orc):
    """fp32 -> fp16 round-to-nearest-even against numpy's float16 cast."""
    rng = np.random.default_rng(7)
    vals = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(3.0),
        (rng.random(20000) * 65504).astype(np.float32),
        np.float32(2.0) ** rng.uniform(-27, -13, 20000).astype(np.float32),   # subnormal range
        np.float32(2.0) ** rng.uniform(-14, 16, 20000).astype(np.float32),
    ])
    # exact ties: fp16 midpoints in the normal and subnormal ranges
    mids = []
    for e in range(-14, 15):
        for m in (0, 1, 2, 511, 1022):
            mids.append((1 + (m + 0.5) / 1024) * 2.0 ** e)
    for k in (0, 1, 2, 3, 1000):
        mids.append((k + 0.5) * 2.0 ** -24)
    vals = np.concatenate([vals, np.array(mids, dtype=np.float32),
                           np.array([65504, 65519, 6.1035156e-05, 5.9604645e-08, 2.9802322e-08],
                                    dtype=np.float32)])
    f = orc.lib().orc_f32_to_f16_rne
    got = np.array([f(float(v)) for v in vals], dtype=np.uint16)
    with np.errstate(over="ignore"):
        want = vals.astype(np.float16).view(np.uint16)
    np.testing.assert_array_equal(got, want)


def test_f16_decode_matches_numpy(orc):
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    finite = (bits & 0x7C00) != 0x7C00
    want = bits[finite].view(np.float16).astype(np.float64)
    got = np.array([orc.f16_to_f64(int(b)) for b in bits[finite]])
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("qmax,n", [(7, 32), (127, 64), (127, 128)])
def test_quantizer_invariants(orc, qmax, n):
    rng = np.random.default_rng(11 + qmax)
    for trial in range(300):
        scale_mag = 2.0 ** rng.uniform(-10, 10)
        x = bf16_bits_from_f32(rng.standard_normal(n).astype(np.float32) * np.float32(scale_mag))
        xf = f32_from_bf16_bits(x).astype(np.float64)
        codes, s = orc.quant_sym(x, qmax)
        s16 = orc.f16_to_f64(s)
        assert np.all(np.abs(codes.astype(int)) <= qmax)
        # the scale is the fp16 rounding of amax / qmax
        amax = np.max(np.abs(xf))
        assert s == np.float16(np.float32(amax) / np.float32(qmax)).view(np.uint16)
        # reconstruction error at most half a step for unclamped codes
        err = np.abs(xf - codes.astype(np.float64) * s16)
        assert np.all(err <= s16 / 2 * (1 + 1e-6) + 1e-300)
        # the largest magnitude maps to +-qmax
        j = int(np.argmax(np.abs(xf)))
        assert abs(int(codes[j])) == qmax


def test_quantizer_scale_only_depends_on_own_values(orc):
    """Calibration-free: a group's codes depend only on that group."""
    rng = np.random.default_rng(5)
    x = bf16_bits_from_f32(rng.standard_normal(32).astype(np.float32))
    a, sa = orc.quant_sym(x, 7)
    b, sb = orc.quant_sym(x.copy(), 7)
    np.testing.assert_array_equal(a, b)
    assert sa == sb
