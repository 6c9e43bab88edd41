"""The C-ABI library loads, exports every declared symbol and rejects bad
arguments on the host before launching anything (runs without a GPU)."""
import ctypes
import os
import re

import pytest

import int4_kv_cache_amd as kv4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kv4.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s+\**([a-z][a-z0-9_]*)\s*\(",
                       src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kv4.LIB_PATH):
        pytest.fail("libkv4.so is not built (python -m int4_kv_cache_amd.build)")
    return kv4.load()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 15, names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in kv4.h but not exported"
    assert set(names) == set(kv4.EXPORTS)


def test_version_and_status_strings(lib):
    assert lib.kv4_abi_version() == 5
    for code, text in kv4.STATUS.items():
        assert lib.kv4_status_string(code).decode() == text
    assert lib.kv4_status_string(12345).decode() == "unknown status"


def test_sizes_closed_form(lib):
    for D in (64, 128):
        lay = kv4.make_layout(32, 8, D, 16, 128)
        assert kv4.block_bytes(kv4.FMT_KV4, lay) == 18 * D
        assert kv4.block_bytes(kv4.FMT_KV8, lay) == 32 * D + 64
        assert kv4.block_bytes(kv4.FMT_BF16, lay) == 64 * D
        assert kv4.side_bytes(lay) == 9 * (32 * D + 64)
    assert kv4.side_bytes(kv4.make_layout(32, 8, 128, 0, 0)) == 0
    assert kv4.block_bytes(kv4.FMT_KV4, kv4.make_layout(32, 8, 96, 0, 0)) == 0


def test_workspace_size(lib):
    lay = kv4.make_layout(32, 8, 128, 16, 128)
    a = kv4.workspace_bytes(lay, 1024, 1040)
    b = kv4.workspace_bytes(lay, 1024, 2080)
    assert 0 < a < b
    with pytest.raises(kv4.Kv4Error) as e:
        kv4.workspace_bytes(lay, 1024, 0)
    assert e.value.status == -1
    with pytest.raises(kv4.Kv4Error) as e:
        kv4.workspace_bytes(kv4.make_layout(32, 8, 96, 0, 0), 4, 4)
    assert e.value.status == -2


def _call_decode(lib, lay, cache, batch, q=1, out=1, ws=1, ws_bytes=1 << 40):
    return lib.kv4_decode_attention(ctypes.byref(lay), ctypes.byref(cache) if cache else None,
                                    ctypes.byref(batch) if batch else None, q, 1.0, out, None, ws,
                                    ws_bytes, None)


def test_host_argument_errors_return_before_launch(lib):
    """Fake (never dereferenced) pointers: each call must fail on the host."""
    good = kv4.make_layout(32, 8, 128, 16, 128)
    fake = 0x1000
    cache = kv4.CacheDesc(fake, 10, fake, 4)
    batch = kv4.BatchDesc(fake, 4, fake, None, 4)
    # bad layouts
    for lay, want in [(kv4.make_layout(32, 7, 128, 16, 128), -1),    # Hq % Hkv
                      (kv4.make_layout(32, 8, 96, 16, 128), -2),     # head_dim
                      (kv4.make_layout(32, 8, 128, 16, 129, flags=0), -1),    # S + R > 144
                      (kv4.make_layout(32, 8, 128, 16, 4081), -1),   # > 4096 even when widened
                      (kv4.make_layout(32, 8, 128, 16, 128, flags=8), -1),    # unknown flag
                      (kv4.make_layout(32, 8, 128, -1, 0), -1),
                      (kv4.make_layout(32, 8, 128, 16, 128, page_size=32), -2),
                      (kv4.make_layout(32, 8, 128, 16, 128, group_size=64), -2),
                      (kv4.make_layout(48, 8, 128, 16, 128), -2)]:  # g = 6
        assert _call_decode(lib, lay, cache, batch) == want
        assert lib.kv4_append(ctypes.byref(lay), ctypes.byref(cache), ctypes.byref(batch),
                              fake, fake, fake, 3, None) == want
    # null structs / pointers
    assert _call_decode(lib, good, None, batch) == -1
    assert _call_decode(lib, good, cache, None) == -1
    assert _call_decode(lib, good, cache, batch, q=None) == -1
    assert _call_decode(lib, good, cache, batch, out=None) == -1
    assert _call_decode(lib, good, cache, batch, ws=None) == -1
    assert _call_decode(lib, good, kv4.CacheDesc(fake, 10, None, 0), batch) == -1   # side needed
    assert _call_decode(lib, good, kv4.CacheDesc(None, 10, fake, 4), batch) == -1
    assert _call_decode(lib, good, cache, kv4.BatchDesc(None, 4, fake, None, 4)) == -1
    assert _call_decode(lib, good, cache, kv4.BatchDesc(fake, 0, fake, None, 4)) == -1
    # softmax scale must be positive and finite
    for sm in (0.0, -1.0, float("inf"), float("nan")):
        assert lib.kv4_decode_attention(ctypes.byref(good), ctypes.byref(cache), ctypes.byref(batch), fake,
                                        sm, fake, None, fake, 1 << 40, None) == -1
    # the integer-query flag: kv4 only; unknown flag bits are rejected
    q8 = kv4.make_layout(32, 8, 128, 16, 128, int8_query=True)
    assert q8.flags == kv4.LAYOUT_INT8_QUERY
    assert _call_decode(lib, q8, cache, batch, ws_bytes=16) == -3
    assert lib.kv8_decode_attention(ctypes.byref(q8), ctypes.byref(cache), ctypes.byref(batch), fake, 1.0, fake,
                                    None, fake, 1 << 40, None) == -2
    assert _call_decode(lib, kv4.make_layout(32, 8, 128, 16, 128, flags=4), cache, batch) == -1
    # wider protection is accepted behind the flag (then the workspace check is reached)
    wide = kv4.make_layout(32, 8, 128, 32, 480)
    assert wide.flags == kv4.LAYOUT_WIDE_PROTECTION
    assert _call_decode(lib, wide, cache, batch, ws_bytes=16) == -3
    assert kv4.side_bytes(wide) == 32 * (32 * 128 + 64)
    # workspace too small
    assert _call_decode(lib, good, cache, batch, ws_bytes=16) == -3
    # append argument errors
    assert lib.kv4_append(ctypes.byref(good), ctypes.byref(cache), ctypes.byref(batch), fake, fake,
                          fake, -1, None) == -1
    assert lib.kv4_append(ctypes.byref(good), ctypes.byref(cache), ctypes.byref(batch), None, fake,
                          fake, 3, None) == -1
    # zero work is a no-op and succeeds without launching
    assert lib.kv4_append(ctypes.byref(good), ctypes.byref(cache), ctypes.byref(batch), None, None,
                          None, 0, None) == 0
    assert _call_decode(lib, good, cache, kv4.BatchDesc(fake, 4, fake, None, 0)) == 0
    # plain INT4 needs no side cache; kv8 / kvbf16 ignore it
    plain = kv4.make_layout(32, 8, 128, 0, 0)
    assert _call_decode(lib, plain, kv4.CacheDesc(fake, 10, None, 0), batch, ws_bytes=16) == -3
    assert lib.kv8_decode_attention(ctypes.byref(good), ctypes.byref(kv4.CacheDesc(fake, 10, None, 0)),
                                    ctypes.byref(batch), fake, 1.0, fake, None, fake, 16, None) == -3
    # phased decode: the mask must select 1..7; a plan alone needs no cache, q or out
    for ph in (0, 8, 0xFFFFFFFF):
        assert lib.kv4_decode_phases(ctypes.byref(good), ctypes.byref(cache), ctypes.byref(batch), fake, 1.0,
                                     fake, None, fake, 1 << 40, ph, None) == -1
    assert lib.kv4_decode_phases(ctypes.byref(good), None, ctypes.byref(batch), None, 1.0, None, None, fake,
                                 16, 1, None) == -3
    assert lib.kv4_decode_phases(ctypes.byref(good), None, ctypes.byref(batch), None, 1.0, None, None, fake,
                                 1 << 40, 2, None) == -1                       # attend needs the cache
    assert lib.kv4_decode_phases(ctypes.byref(good), ctypes.byref(cache), ctypes.byref(batch), None, 1.0,
                                 fake, None, fake, 1 << 40, 2, None) == -1      # attend needs q
    assert lib.kv4_decode_phases(ctypes.byref(good), ctypes.byref(cache), ctypes.byref(batch), fake, 1.0,
                                 None, None, fake, 1 << 40, 4, None) == -1      # merge needs out
    assert lib.kv8_decode_phases(ctypes.byref(good), None, ctypes.byref(kv4.BatchDesc(fake, 4, fake, None, 0)),
                                 None, 1.0, None, None, None, 0, 1, None) == 0  # empty batch
    # append + decode in one call: both calls' checks, before any launch
    def fused(lay=good, c=cache, b=batch, k=fake, total=3, q=fake, out=fake, ws_bytes=1 << 40, ph=7):
        return lib.kv4_append_decode_phases(ctypes.byref(lay), None if c is None else ctypes.byref(c),
                                            ctypes.byref(b), k, fake, fake, total, q, 1.0, out, None, fake,
                                            ws_bytes, ph, None)
    assert fused(lay=kv4.make_layout(32, 8, 96, 16, 128)) == -2     # layout (append check)
    assert fused(k=None) == -1                                       # append needs k_new
    assert fused(total=-1) == -1
    assert fused(ph=0) == -1 and fused(ph=8) == -1                   # decode check
    assert fused(q=None) == -1 and fused(out=None) == -1
    assert fused(ws_bytes=16) == -3
    assert fused(c=None, ph=1) == -1                                 # the cache is required even for a plan
    assert fused(b=kv4.BatchDesc(fake, 4, fake, None, 0)) == 0       # empty batch: nothing to do
    assert lib.kv8_append_decode_phases(ctypes.byref(good), ctypes.byref(cache), ctypes.byref(batch), fake, fake,
                                        fake, 3, fake, 1.0, fake, None, fake, 16, 7, None) == -3
    # probe
    assert lib.kv4_hbm_read_probe(fake, 17, fake, None) == -1
    assert lib.kv4_hbm_read_probe(None, 16, fake, None) == -1


def test_noalloc_rejects_on_the_host(lib):
    """kv4_decode_attention_noalloc checks arguments and the batch's workspace
    size against its fixed scratch before it looks up or touches the device
    (fake pointers, never dereferenced)."""
    fake = 0x1000
    lay = kv4.make_layout(32, 8, 128, 16, 128)
    cache = kv4.CacheDesc(fake, 10, fake, 128)

    def call(batch, q=fake, out=fake, layout=lay):
        return lib.kv4_decode_attention_noalloc(ctypes.byref(layout), ctypes.byref(cache),
                                                ctypes.byref(batch) if batch else None, q, 1.0, out, None, None)

    # 128 sequences with page tables of 1,040 columns need about 72 MB of workspace
    big = kv4.BatchDesc(fake, 1040, fake, None, 128)
    assert kv4.workspace_bytes(lay, 128, 1040) > kv4.NOALLOC_SCRATCH_BYTES
    assert call(big) == -3
    # the size that still fits is the one kv4_decode_workspace_size reports
    n_fit = max(b for b in range(1, 200) if kv4.workspace_bytes(lay, b, 1040) <= kv4.NOALLOC_SCRATCH_BYTES)
    assert call(kv4.BatchDesc(fake, 1040, fake, None, n_fit + 1)) == -3
    assert 100 <= n_fit < 128
    assert call(None) == -1
    assert call(kv4.BatchDesc(fake, 4, fake, None, 2), q=None) == -1
    assert call(kv4.BatchDesc(fake, 4, fake, None, 2), out=None) == -1
    assert call(kv4.BatchDesc(fake, 0, fake, None, 2)) == -1
    assert call(kv4.BatchDesc(fake, 4, fake, None, 2), layout=kv4.make_layout(32, 8, 96, 0, 0)) == -2
    # an empty batch is a no-op that needs no device
    assert call(kv4.BatchDesc(None, 4, None, None, 0)) == 0
