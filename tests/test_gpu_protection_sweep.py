"""Protection-width sweep at the Qwen3-8B-shaped layer (B=1024): KV4-RL with
(sinks, recent) in {(0,0), (4,16), (16,64), (16,128), (16,256), (32,480)} on
identical seeded K/V.  Widths beyond the method's 144 use the layout flag
KV4_LAYOUT_WIDE_PROTECTION.  For every width: cache bytes bit-exact and
outputs within the parity bounds on a sample, decode time (HIP events), and
the attention KL against BF16 in the oracle.  The protected sets are nested,
so the mean KL must not grow with the width (INT8 rows replace INT4 rows)."""
import gc

import numpy as np
import pytest

import parity_util as pu

pytestmark = pytest.mark.gpu

WIDTHS = [(0, 0), (4, 16), (16, 64), (16, 128), (16, 256), (32, 480)]
N_KL = 32
N_PARITY = 8


def _time_decode(wl, n=10):
    import torch

    for _ in range(3):
        wl.decode()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        wl.decode()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n * 1e3


def test_protection_width_sweep(kv4):
    import oracle
    import torch

    from harness import build_config

    gc.collect()
    torch.cuda.empty_cache()
    rng = np.random.default_rng(55)
    sample = np.sort(rng.choice(1024, size=N_KL, replace=False))
    psample = sample[:N_PARITY]
    ref = build_config(2, kv4.FMT_BF16, keep_inputs=True)
    ref.step_append()
    rcache, rpt, rlens = pu.oracle_cache_for(ref, sample)
    q = (ref.host_q()[sample].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    lay = ref.layout
    g = lay.num_q_heads // lay.num_kv_heads
    Kref = [[oracle.gather(rcache, rpt, rlens, None, i, h)[0] for h in range(lay.num_kv_heads)]
            for i in range(len(sample))]
    del ref
    rows = []
    for S, R in WIDTHS:
        wl = build_config(2, kv4.FMT_KV4, n_sink=S, n_recent=R, keep_inputs=True)
        wl.step_append()
        us = _time_decode(wl)
        ocache, pt, lens = pu.compare_bytes(wl, psample)
        m = pu.decode_metrics(wl, psample, ocache, pt, lens)
        pu.assert_within(m)
        vcache, vpt, vlens = pu.oracle_cache_for(wl, sample)
        kls = []
        for i in range(len(sample)):
            for h in range(lay.num_kv_heads):
                Kv = oracle.gather(vcache, vpt, vlens, None, i, h)[0]
                for j in range(g):
                    pr = oracle.probs(q[i, h * g + j], Kref[i][h])
                    pv = oracle.probs(q[i, h * g + j], Kv)
                    kls.append(float(np.sum(pr * (np.log(pr) - np.log(pv)))))
        rows.append((S, R, us, float(np.mean(kls)), float(np.max(kls)), m))
        print(f"protection S={S:3d} R={R:3d}: decode {us:7.1f} us  KL mean {rows[-1][3]:.4e} max {rows[-1][4]:.4e}  "
              f"parity rel_l2={m['rel_l2']:.2e} lse={m['lse_abs']:.2e}", flush=True)
        del wl
        gc.collect()
        torch.cuda.empty_cache()
    means = [r[3] for r in rows]
    for a, b in zip(means, means[1:]):
        assert b <= a * 1.02, means
