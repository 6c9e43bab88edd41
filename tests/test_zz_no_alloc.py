"""kv4_decode_attention_noalloc (the decode with the library's fixed per-GPU
scratch instead of a caller workspace) against kv4_decode_attention, through
the C ABI: the same bits on two calls in a row, the second over a smaller
batch, and the oracle's bounds on the first; a batch too large for the
scratch is rejected before anything runs."""
import numpy as np
import pytest

import parity_util as pu

pytestmark = pytest.mark.gpu


def _workload(lengths):
    from harness import build_config

    import int4_kv_cache_amd as lib

    wl = build_config(1, lib.FMT_KV4, keep_inputs=True, lengths=np.asarray(lengths, dtype=np.int32))
    wl.step_append()
    return wl


def _same_as_workspace_decode(kv4, wl, label):
    import torch

    wl.decode()
    torch.cuda.synchronize()
    ref_out, ref_lse = wl.out.clone(), wl.lse.clone()
    out = torch.full_like(wl.out, float("nan"))
    lse = torch.full_like(wl.lse, float("nan"))
    print(f"\nnoalloc {label}: batch {wl.lengths.size}, max_pages {wl.alloc.max_pages}, workspace need "
          f"{kv4.workspace_bytes(wl.layout, wl.lengths.size, wl.alloc.max_pages)} B", flush=True)
    kv4.decode_noalloc(wl.cache, wl.batch, wl.q, out, lse)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), label
    assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32)), label
    return out, lse


def test_noalloc_matches_workspace_decode_twice(kv4):
    import torch

    from workloads import context_lengths, get_config

    lens = context_lengths(get_config(1))
    # first call: 100 sequences (long ones split over several items: partials
    # and the merge run in the scratch); second call: 24 shorter sequences
    first = np.sort(lens)[::-1][:100]
    second = np.sort(lens)[:24]
    a = _workload(first)
    out, lse = _same_as_workspace_decode(kv4, a, "first call")
    assert np.any(a.lengths > 16 * 64), "some sequences are split"
    # the oracle's bounds on the no-alloc output itself
    a.out.copy_(out)
    a.lse.copy_(lse)
    sample = np.unique(np.concatenate([np.arange(6), np.arange(94, 100), np.arange(10, 90, 13)]))
    ocache, pt, ol = pu.compare_bytes(a, sample)
    m = pu.decode_metrics(a, sample, ocache, pt, ol)
    print(f"  oracle: rel_l2={m['rel_l2']:.3e} max_abs={m['max_abs']:.3e} lse={m['lse_abs']:.3e}", flush=True)
    pu.assert_within(m)
    b = _workload(second)
    _same_as_workspace_decode(kv4, b, "second call, smaller batch")
    # and the first batch again, after the smaller one left its plan behind
    _same_as_workspace_decode(kv4, a, "third call, first batch again")


def test_noalloc_rejects_a_batch_too_large(kv4):
    import torch

    from harness import build_config
    from workloads import context_lengths, get_config

    # config 1's 128 sequences with one at the 16,640-token cap: page tables
    # of 1,040 columns, about 72 MB of workspace
    lens = context_lengths(get_config(1)).copy()
    lens[0] = 16640
    wl = build_config(1, kv4.FMT_KV4, lengths=lens)
    need = kv4.workspace_bytes(wl.layout, wl.lengths.size, wl.alloc.max_pages)
    assert need > kv4.NOALLOC_SCRATCH_BYTES
    out = torch.full_like(wl.out, 7.0)
    with pytest.raises(kv4.Kv4Error) as e:
        kv4.decode_noalloc(wl.cache, wl.batch, wl.q, out, wl.lse)
    assert e.value.status == -3
    torch.cuda.synchronize()
    assert torch.all(out == 7.0), "nothing was launched"
