"""Config 3 at full size: 36 Qwen3-8B-shaped layers, 512 sequences with
contexts uniform in [4096, 16600] (about 226 GB of INT4 pages and INT8 side
caches resident), decoded the way bench.py --config 3 times it (one plan,
attend + merge per layer).  A seeded sample of sequences is checked in every
layer: cache bytes bit-exact, outputs within the parity bounds."""
import gc

import numpy as np
import pytest

import parity_util as pu

pytestmark = pytest.mark.gpu

N_SAMPLE = 12


def test_config3_36_layers_sampled(kv4):
    import torch

    from harness import build_layers

    gc.collect()
    torch.cuda.empty_cache()
    wl = build_layers(3, kv4.FMT_KV4,
                      progress=lambda l: print(f"layer {l} built", flush=True) if l % 6 == 5 else None)
    try:
        wl.step()
        torch.cuda.synchronize()
        sample = np.sort(np.random.default_rng(33).choice(wl.lengths.size, size=N_SAMPLE, replace=False))
        worst = dict(rel_l2=0.0, max_abs=0.0, lse_abs=0.0)
        for l in range(wl.n_layers):
            view = wl.layer(l)
            wl.want(l, sample)
            ocache, pt, lens = pu.compare_bytes(view, sample)
            m = pu.decode_metrics(view, sample, ocache, pt, lens)
            for k in worst:
                worst[k] = max(worst[k], m[k])
            print(f"config3 layer {l}: rel_l2={m['rel_l2']:.3e} max_abs={m['max_abs']:.3e} "
                  f"lse={m['lse_abs']:.3e}", flush=True)
            pu.assert_within(m)
        print(f"config3 worst over 36 layers x {N_SAMPLE} sequences: {worst}", flush=True)
    finally:
        del wl
        gc.collect()
        torch.cuda.empty_cache()
