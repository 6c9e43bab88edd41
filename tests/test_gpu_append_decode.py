"""kv4_append_decode_phases (append, then the decode phases, with the plan in
the append's launch) against kv4_append followed by kv4_decode_phases: the
same page and side-cache bytes and the same out / lse bits, for every format,
for the phases split over several calls, and for a ragged append in which
only some sequences receive a token."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

ALL = 7


def _state(wl):
    side = wl.cache.side.clone() if getattr(wl.cache, "side", None) is not None else None
    return wl.cache.pages.clone(), side


def _restore(wl, st):
    wl.cache.pages.copy_(st[0])
    if st[1] is not None:
        wl.cache.side.copy_(st[1])


def _same(wl, ref, out, lse):
    import torch

    torch.cuda.synchronize()
    assert torch.equal(wl.cache.pages, ref["pages"])
    if ref["side"] is not None:
        assert torch.equal(wl.cache.side, ref["side"])
    assert torch.equal(out.view(torch.int16), ref["out"].view(torch.int16))
    assert torch.equal(lse.view(torch.int32), ref["lse"].view(torch.int32))


@pytest.mark.parametrize("fmt,q8", [(0, False), (0, True), (1, False), (2, False)],
                         ids=["kv4", "kv4-int8q", "kv8", "bf16"])
def test_fused_matches_separate_calls(kv4, fmt, q8):
    import torch

    from harness import build_config

    wl = build_config(1, fmt, int8_query=q8)
    before = _state(wl)
    print(f"\nfused append+decode fmt={fmt} q8={q8} batch={wl.lengths.size}", flush=True)

    def run_case(k, v, cu):
        # reference: the two calls
        _restore(wl, before)
        kv4.append(wl.cache, wl.batch, k, v, cu)
        kv4.decode_phases(wl.cache, wl.batch, wl.q, wl.out, wl.lse, wl.workspace, ALL)
        torch.cuda.synchronize()
        ref = {"pages": wl.cache.pages.clone(), "out": wl.out.clone(), "lse": wl.lse.clone(),
               "side": wl.cache.side.clone() if before[1] is not None else None}
        ws = torch.empty_like(wl.workspace)
        # one call, all phases
        for split in ("one call", "plan fused, attend and merge apart", "plan apart, append with attend"):
            _restore(wl, before)
            ws.fill_(0xA5)
            out = torch.full_like(wl.out, float("nan"))
            lse = torch.full_like(wl.lse, float("nan"))
            if split == "one call":
                kv4.append_decode_phases(wl.cache, wl.batch, k, v, cu, wl.q, out, lse, ws, ALL)
            elif split == "plan fused, attend and merge apart":
                kv4.append_decode_phases(wl.cache, wl.batch, k, v, cu, None, None, None, ws, kv4.PHASE_PLAN)
                kv4.decode_phases(wl.cache, wl.batch, wl.q, out, lse, ws, kv4.PHASE_ATTEND)
                kv4.decode_phases(wl.cache, wl.batch, wl.q, out, lse, ws, kv4.PHASE_MERGE)
            else:
                kv4.decode_phases(wl.cache, wl.batch, None, None, None, ws, kv4.PHASE_PLAN)
                kv4.append_decode_phases(wl.cache, wl.batch, k, v, cu, wl.q, out, lse, ws,
                                         kv4.PHASE_ATTEND | kv4.PHASE_MERGE)
            _same(wl, ref, out, lse)
            print(f"  {split}: identical", flush=True)

    # every sequence appends its step token
    run_case(wl.step_k, wl.step_v, wl.step_cu)
    # ragged: only every third sequence appends (the others keep what the pages hold)
    B = wl.lengths.size
    keep = np.arange(B) % 3 == 0
    cu = np.concatenate([[0], np.cumsum(keep)]).astype(np.int32)
    idx = torch.from_numpy(np.flatnonzero(keep)).to("cuda")
    run_case(wl.step_k[idx].contiguous(), wl.step_v[idx].contiguous(), torch.from_numpy(cu).to("cuda"))
    # nothing to append: the decode alone
    _restore(wl, before)
    kv4.decode_phases(wl.cache, wl.batch, wl.q, wl.out, wl.lse, wl.workspace, ALL)
    torch.cuda.synchronize()
    ref_out, ref_lse = wl.out.clone(), wl.lse.clone()
    out = torch.full_like(wl.out, float("nan"))
    lse = torch.full_like(wl.lse, float("nan"))
    empty = torch.zeros((0,) + tuple(wl.step_k.shape[1:]), dtype=wl.step_k.dtype, device="cuda")
    kv4.append_decode_phases(wl.cache, wl.batch, empty, empty, torch.zeros(B + 1, dtype=torch.int32,
                                                                              device="cuda"),
                             wl.q, out, lse, wl.workspace, ALL)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32))
    assert torch.equal(wl.cache.pages, before[0])


@pytest.mark.parametrize("fmt", [0, 1], ids=["kv4", "kv8"])
def test_fused_multi_token_reappend(kv4, fmt):
    """Several tokens per sequence in one fused call: the last three positions
    of every sequence appended again (host-built cache, so the tokens are
    known) leave every page and side byte unchanged, and the decode matches
    the separate decode bit for bit."""
    import torch

    from harness import build_from_host
    from harness.device import _bf16, _i32

    wl = build_from_host(0, fmt)
    wl.decode()
    torch.cuda.synchronize()
    ref_out, ref_lse = wl.out.clone(), wl.lse.clone()
    pages = wl.cache.pages.clone()
    side = wl.cache.side.clone() if getattr(wl.cache, "side", None) is not None else None
    n_b = np.minimum(wl.lengths, 3)
    ks = [wl.tokens["host_k"][b][wl.lengths[b] - n_b[b]:] for b in range(wl.lengths.size)]
    vs = [wl.tokens["host_v"][b][wl.lengths[b] - n_b[b]:] for b in range(wl.lengths.size)]
    k_new = _bf16(np.concatenate(ks), "cuda")
    v_new = _bf16(np.concatenate(vs), "cuda")
    cu = _i32(np.concatenate([[0], np.cumsum(n_b)]), "cuda")
    print(f"\nre-append {int(n_b.sum())} tokens over {wl.lengths.size} sequences, fmt={fmt}", flush=True)
    out = torch.full_like(wl.out, float("nan"))
    lse = torch.full_like(wl.lse, float("nan"))
    ws = torch.empty_like(wl.workspace)
    ws.fill_(0x33)
    kv4.append_decode_phases(wl.cache, wl.batch, k_new, v_new, cu, wl.q, out, lse, ws)
    torch.cuda.synchronize()
    assert torch.equal(wl.cache.pages, pages)
    if side is not None:
        assert torch.equal(wl.cache.side, side)
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32))


@pytest.mark.parametrize("fmt,q8", [(0, False), (0, True), (1, False), (2, False)],
                         ids=["kv4", "kv4-int8q", "kv8", "bf16"])
def test_fused_step_against_oracle(kv4, fmt, q8):
    """The fused call itself against the oracle (not only against the other
    HIP calls): config 1, every sequence appends its step token and the plan
    shares the append's launch; then the page and side bytes of every
    sequence, including the appended tokens, and every output."""
    import torch

    import parity_util as pu
    from harness import build_config

    wl = build_config(1, fmt, int8_query=q8, keep_inputs=True)
    print(f"\nfused step vs oracle fmt={fmt} q8={q8} batch={wl.lengths.size}", flush=True)
    ws = torch.empty_like(wl.workspace)
    ws.fill_(0x3C)
    kv4.append_decode_phases(wl.cache, wl.batch, wl.step_k, wl.step_v, wl.step_cu, wl.q, wl.out, wl.lse, ws, ALL)
    torch.cuda.synchronize()
    sample = np.arange(wl.lengths.size)
    ocache, pt, lens = pu.compare_bytes(wl, sample)
    m = pu.decode_metrics(wl, sample, ocache, pt, lens)
    print(f"  rel_l2={m['rel_l2']:.3e} max_abs={m['max_abs']:.3e} lse={m['lse_abs']:.3e}", flush=True)
    pu.assert_within(m)
