"""Helpers for comparing the GPU library with the CPU oracle.

The oracle rebuilds the cache of a sample of sequences from the same seeded
bf16 inputs; its bytes must equal the GPU's bytes exactly.  Decode outputs are
then compared with the oracle evaluated on those (identical) bytes:
  * rel_l2  = ||out_gpu - bf16(out64)|| / ||bf16(out64)||   (bound 1e-3)
  * max_abs = max |out_gpu - out64|                          (bound 1e-2)
  * lse     : max |lse_gpu - lse64|                          (bound 1e-4)
The bf16 output rounding alone is ~1.6e-3 relative RMS against fp64, so the
relative bound is taken against the oracle rounded to bf16 (nearest even).
"""
from __future__ import annotations

import numpy as np

import oracle

REL_L2_MAX = 1e-3
MAX_ABS_MAX = 1e-2
LSE_ABS_MAX = 1e-4


def to_bf16_rne(x: np.ndarray) -> np.ndarray:
    """fp64 -> nearest bf16 value (8 significant bits, ties to even), as fp64."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                      # x = m * 2^e, |m| in [0.5, 1)
    return np.ldexp(np.rint(m * 256.0), e - 8)


def bf16_bits_to_f64(b) -> np.ndarray:
    u = np.ascontiguousarray(b).view(np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def torch_u8(t) -> np.ndarray:
    return t.cpu().numpy()


def oracle_cache_for(wl, sample):
    """Oracle cache of the sampled sequences, compact page ids, slot = index."""
    lay = oracle.make_layout(wl.layout.num_q_heads, wl.layout.num_kv_heads, wl.layout.head_dim,
                             wl.layout.n_sink, wl.layout.n_recent)
    fmt = {0: oracle.FMT_KV4, 1: oracle.FMT_KV8, 2: oracle.FMT_BF16}[wl.fmt]
    lens = wl.lengths[sample].astype(np.int32)
    npg = (lens + 15) // 16
    mp = int(max(1, npg.max(initial=1)))
    pt = np.zeros((len(sample), mp), dtype=np.int32)
    nxt = 0
    for i, n in enumerate(npg):
        pt[i, :n] = np.arange(nxt, nxt + n)
        nxt += int(n)
    cache = oracle.HostCache(fmt, lay, max(1, nxt), len(sample))
    ks, vs = [], []
    for b in sample:
        k, v = wl.host_tokens(int(b))
        ks.append(k)
        vs.append(v)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    if cu[-1] > 0:
        oracle.append(cache, pt, lens, None, np.concatenate(ks), np.concatenate(vs), cu)
    return cache, pt, lens


def gpu_cache_bytes(wl, sample, pt_compact):
    """The GPU's pages/side blocks of the sample, in the oracle's compact order."""
    import torch

    H = wl.layout.num_kv_heads
    bb = wl.cache.pages.numel() // (wl.cache.num_pages * H)
    pool = wl.cache.pages.view(wl.cache.num_pages, H * bb)
    lens = wl.lengths[sample]
    npg = (lens + 15) // 16
    phys = np.concatenate([wl.alloc.page_table[b, :n] for b, n in zip(sample, npg)]) if npg.sum() else \
        np.zeros(0, np.int64)
    pages = pool[torch.as_tensor(phys.astype(np.int64), device=pool.device)].cpu().numpy().ravel()
    side = None
    if wl.cache.side is not None:
        slots = wl.tokens.get("slots")
        idx = np.asarray(sample) if slots is None else slots[np.asarray(sample)]
        sb = wl.cache.side.numel() // wl.cache.num_slots
        sv = wl.cache.side.view(wl.cache.num_slots, sb)
        side = sv[torch.as_tensor(idx.astype(np.int64), device=sv.device)].cpu().numpy().ravel()
    return pages, side


def valid_side_rows_mask(wl, sample):
    """Byte mask of side-cache rows that hold live positions (others are
    undefined scratch and not compared)."""
    lay = wl.layout
    S, R, D, H = lay.n_sink, lay.n_recent, lay.head_dim, lay.num_kv_heads
    rows = S + R
    tiles = (rows + 15) // 16
    tile_b = 32 * D + 64
    sb = tiles * tile_b
    masks = []
    for b in sample:
        L = int(wl.lengths[b])
        live = set()
        for p in range(min(S, L)):
            live.add(p)
        for p in range(max(S, L - R), L):
            live.add(S + (p - S) % R)
        m = np.zeros(sb, dtype=bool)
        for rho in live:
            t, r = divmod(rho, 16)
            base = t * tile_b
            m[base + r * D: base + (r + 1) * D] = True                       # K codes
            q4, rr = divmod(r, 4)
            for c in range(D):                                               # V codes
                m[base + 16 * D + (q4 * 16 + c % 16) * (D // 4) + (c // 16) * 4 + rr] = True
            m[base + 32 * D + 2 * r: base + 32 * D + 2 * r + 2] = True         # K scale
            m[base + 32 * D + 32 + 2 * r: base + 32 * D + 32 + 2 * r + 2] = True
        masks.append(np.tile(m, H))
    return np.concatenate(masks) if masks else np.zeros(0, bool)


def compare_bytes(wl, sample):
    """Assert the GPU's cache bytes of the sample equal the oracle's."""
    ocache, pt, lens = oracle_cache_for(wl, sample)
    pages, side = gpu_cache_bytes(wl, sample, pt)
    n = pages.size
    np.testing.assert_array_equal(pages, ocache.pages[:n], err_msg="page bytes differ from the oracle")
    if side is not None:
        mask = valid_side_rows_mask(wl, sample)
        np.testing.assert_array_equal(side[mask], ocache.side[:side.size][mask],
                                      err_msg="side-cache bytes differ from the oracle")
    return ocache, pt, lens


def decode_metrics(wl, sample, ocache=None, pt=None, lens=None, nthreads=0):
    """Oracle decode of the sample vs the GPU output; returns a dict."""
    if ocache is None:
        ocache, pt, lens = oracle_cache_for(wl, sample)
    q = wl.host_q()[np.asarray(sample)]
    q_int8 = bool(wl.layout.flags & 2)   # the integer-query layout flag
    out64, lse64, gap = oracle.decode(ocache, pt, lens, None, np.ascontiguousarray(q), 1.0,
                                      nthreads=nthreads, q_int8=q_int8)
    import torch

    og = bf16_bits_to_f64(wl.out.view(torch.int16).cpu().numpy()[np.asarray(sample)])
    lg = wl.lse.cpu().numpy().astype(np.float64)[np.asarray(sample)]
    ref = to_bf16_rne(out64)
    denom = np.linalg.norm(ref)
    rel = float(np.linalg.norm(og - ref) / denom) if denom > 0 else float(np.linalg.norm(og - ref))
    max_abs = float(np.max(np.abs(og - out64))) if og.size else 0.0
    fin = np.isfinite(lse64)
    assert np.array_equal(fin, np.isfinite(lg)), "lse finiteness differs"
    lse_err = float(np.max(np.abs(lg[fin] - lse64[fin]))) if fin.any() else 0.0
    # and the other way round, for information
    rel64 = float(np.linalg.norm(og - out64) / max(np.linalg.norm(out64), 1e-300))
    return dict(rel_l2=rel, max_abs=max_abs, lse_abs=lse_err, rel_l2_vs_fp64=rel64, merge_gap=gap,
                n=len(sample))


def metrics_from(og, lg, out64, lse64, gap):
    """Bounds of the module docstring for GPU outputs og (bf16 values as fp64)
    and lse lg against oracle out64 / lse64 of the same shape."""
    ref = to_bf16_rne(out64)
    denom = np.linalg.norm(ref)
    rel = float(np.linalg.norm(og - ref) / denom) if denom > 0 else float(np.linalg.norm(og - ref))
    max_abs = float(np.max(np.abs(og - out64))) if og.size else 0.0
    fin = np.isfinite(lse64)
    assert np.array_equal(fin, np.isfinite(lg)), "lse finiteness differs"
    lse_err = float(np.max(np.abs(lg[fin] - lse64[fin]))) if fin.any() else 0.0
    rel64 = float(np.linalg.norm(og - out64) / max(np.linalg.norm(out64), 1e-300))
    return dict(rel_l2=rel, max_abs=max_abs, lse_abs=lse_err, rel_l2_vs_fp64=rel64, merge_gap=gap,
                n=int(out64.shape[0]))


def assert_within(m):
    assert m["rel_l2"] <= REL_L2_MAX, m
    assert m["max_abs"] <= MAX_ABS_MAX, m
    assert m["lse_abs"] <= LSE_ABS_MAX, m
    assert m["merge_gap"] <= 1e-12, m
