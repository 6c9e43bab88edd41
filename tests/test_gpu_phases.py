"""Phased decode through the C ABI: PLAN once, then ATTEND + MERGE for two
layers that share the page table and seq_lens, must give the same bits as a
full decode call per layer; and the phased result passes the oracle check."""
import numpy as np
import pytest

import parity_util as pu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt", [0, 1, 2], ids=["kv4", "kv8", "bf16"])
def test_plan_reused_across_layers(kv4, fmt):
    import torch

    from harness import build_config

    layers = [build_config(1, fmt, layer=l, keep_inputs=(l == 1)) for l in (0, 1)]
    for wl in layers:
        wl.step_append()
    assert np.array_equal(layers[0].lengths, layers[1].lengths)
    refs = []
    for wl in layers:
        wl.decode()
        torch.cuda.synchronize()
        refs.append((wl.out.clone(), wl.lse.clone()))
    ws = torch.empty_like(layers[0].workspace)
    ws.fill_(0xA5)  # the plan must not depend on earlier workspace contents
    w0 = layers[0]
    kv4.decode_phases(w0.cache, w0.batch, None, None, None, ws, kv4.PHASE_PLAN)
    for wl, (ref_out, ref_lse) in zip(layers, refs):
        out = torch.full_like(wl.out, float("nan"))
        lse = torch.full_like(wl.lse, float("nan"))
        kv4.decode_phases(wl.cache, wl.batch, wl.q, out, lse, ws, kv4.PHASE_ATTEND)
        kv4.decode_phases(wl.cache, wl.batch, wl.q, out, lse, ws, kv4.PHASE_MERGE)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
        assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32))
    # the second layer's phased output against the oracle on a sample
    wl = layers[1]
    wl.out.copy_(out)
    wl.lse.copy_(lse)
    sample = np.random.default_rng(5).choice(wl.lengths.size, size=16, replace=False)
    ocache, pt, lens = pu.oracle_cache_for(wl, np.sort(sample))
    m = pu.decode_metrics(wl, np.sort(sample), ocache, pt, lens)
    print(f"\nphased layer-1 parity fmt={fmt}: rel_l2={m['rel_l2']:.3e} max_abs={m['max_abs']:.3e} "
          f"lse={m['lse_abs']:.3e}", flush=True)
    pu.assert_within(m)


@pytest.mark.parametrize("fmt", [0, 1], ids=["kv4", "kv8"])
def test_attend_repeated_on_one_plan(kv4, fmt):
    """A plan is read, never consumed, by the attention phase (the per-CU
    ticket counters live in LDS and start at zero in every launch; the last
    wave of a launch zeroes the device counter of the list's tail): many
    ATTEND + MERGE pairs on one PLAN, with different queries in between, each
    give the bits of a full decode."""
    import torch

    from harness import build_config

    wl = build_config(1, fmt)
    wl.step_append()
    ws = torch.empty_like(wl.workspace)
    ws.fill_(0x5A)
    kv4.decode_phases(wl.cache, wl.batch, None, None, None, ws, kv4.PHASE_PLAN)
    gen = torch.Generator(device="cpu").manual_seed(11)
    for rep in range(6):
        q = (torch.randn(wl.q.shape, generator=gen) * (1 + rep)).to(torch.bfloat16).to("cuda")
        wl.q.copy_(q)
        wl.decode()
        torch.cuda.synchronize()
        ref_out, ref_lse = wl.out.clone(), wl.lse.clone()
        out = torch.full_like(wl.out, float("nan"))
        lse = torch.full_like(wl.lse, float("nan"))
        kv4.decode_phases(wl.cache, wl.batch, wl.q, out, lse, ws, kv4.PHASE_ATTEND)
        kv4.decode_phases(wl.cache, wl.batch, wl.q, out, lse, ws, kv4.PHASE_MERGE)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), rep
        assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32)), rep


@pytest.mark.parametrize("fmt", [0, 2], ids=["kv4", "bf16"])
def test_attend_twice_without_merge(kv4, fmt):
    """ATTEND with one query, ATTEND again with another, then MERGE: the
    result is the second query's full decode, bit for bit.  Every unit of the
    second launch must run, including those of the list's tail, which are
    drawn from a device counter that the first launch's last wave resets; a
    unit that did not run would keep the first query's values."""
    import torch

    from harness import build_config

    wl = build_config(1, fmt)
    wl.step_append()
    ws = torch.empty_like(wl.workspace)
    ws.fill_(0x5A)
    kv4.decode_phases(wl.cache, wl.batch, None, None, None, ws, kv4.PHASE_PLAN)
    header = ws[:16].view(torch.int32).cpu()
    nitems, cus = int(header[1]), torch.cuda.get_device_properties(0).multi_processor_count
    assert nitems - (nitems - nitems // 4) // cus * cus > 0, "the workload has no tail"
    gen = torch.Generator(device="cpu").manual_seed(12)
    q1 = (torch.randn(wl.q.shape, generator=gen) * 3).to(torch.bfloat16).to("cuda")
    q2 = torch.randn(wl.q.shape, generator=gen).to(torch.bfloat16).to("cuda")
    wl.q.copy_(q2)
    wl.decode()
    torch.cuda.synchronize()
    ref_out, ref_lse = wl.out.clone(), wl.lse.clone()
    out = torch.full_like(wl.out, float("nan"))
    lse = torch.full_like(wl.lse, float("nan"))
    kv4.decode_phases(wl.cache, wl.batch, q1, out, lse, ws, kv4.PHASE_ATTEND)
    kv4.decode_phases(wl.cache, wl.batch, q2, out, lse, ws, kv4.PHASE_ATTEND)
    kv4.decode_phases(wl.cache, wl.batch, q2, out, lse, ws, kv4.PHASE_MERGE)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32))
