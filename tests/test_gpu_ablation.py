"""Config 4, precision ablation at the config-2 shapes: BF16-KV, all-INT8-KV,
plain INT4-KV (no protection), KV4-RL (INT4 + 16 sink / 128 recent INT8
rows) and KV4-RL with the integer query (INT8-quantized q) on identical
seeded K/V.  Each variant's GPU output is compared with
the GPU BF16 output (max-abs over every (sequence, query head)), and the
attention distributions of a seeded sample of 128 sequences are compared
with BF16's in the oracle (KL(pi_bf16 || pi_variant), fp64).

The checks are the orderings the quantization must produce: INT8 keys are
closer to BF16 than INT4 ones, and replacing INT4 by INT8 at the protected
positions can only shrink the deviation on average.  The numbers themselves
are reported, not pinned (the pages' accuracy figures are end-to-end model
scores, not per-kernel deviations)."""
import gc

import numpy as np
import pytest

import parity_util as pu

pytestmark = pytest.mark.gpu

N_KL = 128


def _kl_stats(wls, sample):
    import oracle

    caches = {name: pu.oracle_cache_for(wl, sample) for name, wl in wls.items()}
    qbits = wls["bf16"].host_q()[sample]
    qf = (qbits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)   # [n][Hq][D]
    lay = wls["bf16"].layout
    g = lay.num_q_heads // lay.num_kv_heads
    kl = {name: [] for name in wls if name != "bf16"}
    for i in range(len(sample)):
        for h in range(lay.num_kv_heads):
            Ks = {}
            for name, (oc, pt, lens) in caches.items():
                Ks[name] = oracle.gather(oc, pt, lens, None, i, h)[0]
            for j in range(g):
                hq = h * g + j
                p_ref = oracle.probs(qf[i, hq], Ks["bf16"])
                for name in kl:
                    qv = qf[i, hq]
                    if wls[name].layout.flags & 2:   # integer query: q -> INT8 row codes x scale
                        codes, sbits = oracle.quant_sym(qbits[i, hq], 127)
                        qv = codes.astype(np.float64) * oracle.f16_to_f64(int(sbits))
                    p = oracle.probs(qv, Ks[name])
                    kl[name].append(float(np.sum(p_ref * (np.log(p_ref) - np.log(p)))))
    return {name: (float(np.mean(v)), float(np.max(v))) for name, v in kl.items()}


def test_config4_precision_ablation(kv4):
    import torch

    from harness import build_config

    gc.collect()
    torch.cuda.empty_cache()
    variants = {"bf16": (kv4.FMT_BF16, None, None, False), "kv8": (kv4.FMT_KV8, None, None, False),
                "int4_plain": (kv4.FMT_KV4, 0, 0, False), "kv4_rl": (kv4.FMT_KV4, None, None, False),
                "kv4_rl_q8": (kv4.FMT_KV4, None, None, True)}
    wls = {}
    try:
        for name, (fmt, S, R, q8) in variants.items():
            wl = build_config(4, fmt, n_sink=S, n_recent=R, keep_inputs=True, int8_query=q8)
            wl.step_append()
            wl.decode()
            torch.cuda.synchronize()
            wls[name] = wl
        ref = wls["bf16"].out.float()
        maxabs = {name: float((wl.out.float() - ref).abs().max()) for name, wl in wls.items() if name != "bf16"}
        sample = np.sort(np.random.default_rng(44).choice(ref.shape[0], size=N_KL, replace=False))
        kl = _kl_stats(wls, sample)
        for name in maxabs:
            print(f"config4 {name}: max_abs_vs_bf16={maxabs[name]:.4e} attention_KL mean={kl[name][0]:.4e} "
                  f"max={kl[name][1]:.4e}", flush=True)
        assert maxabs["kv8"] < maxabs["int4_plain"] and maxabs["kv8"] < maxabs["kv4_rl"]
        assert kl["kv8"][0] < kl["kv4_rl"][0] < kl["int4_plain"][0]
    finally:
        wls.clear()
        gc.collect()
        torch.cuda.empty_cache()
