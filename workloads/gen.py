"""Seeded generators: context lengths, bf16 K/V/q draws, page tables.

Recipe (every choice here is an input distribution, not part of the method):
  * lengths   numpy default_rng([seed, 777]); response ~ rint(lognormal(mu,
              sigma)) with mu = ln(mean) - sigma^2/2 so the mean is `mean`,
              clipped to [1, cap]; context = prompt + response.  Uniform
              configs draw integers in [lo, hi].
  * outliers  default_rng([seed, 999]) picks n_outlier key channels; those
              channels of K are multiplied by 8 (the same channels for every
              head, layer and token).
  * host data default_rng([seed, layer, b]) per sequence, draw order K, V, q;
              a shared prompt comes from default_rng([seed, layer, 10**6 +
              group]).  K, V ~ N(0, 1), q ~ N(0, 1) / sqrt(D); fp32 draws
              rounded to bf16 (nearest, ties to even).
  * device    for the large workloads the same distributions are drawn with a
              torch generator on the GPU, seeded from (seed, layer, stream).
  * pages     physical page ids are a seeded permutation, so logically
              consecutive pages are scattered in the pool.
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

from .configs import Config


# --------------------------------------------------------------- bf16 bits ---
def bf16_bits_from_f32(x) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return bits."""
    a = np.ascontiguousarray(x, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounding = ((u >> 16) & 1) + 0x7FFF
    return ((u + rounding) >> 16).astype(np.uint16)


def f32_from_bf16_bits(b) -> np.ndarray:
    u = np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32)


# ----------------------------------------------------------------- lengths ---
def context_lengths(cfg: Config) -> np.ndarray:
    if cfg.fixed_lengths is not None:
        return np.asarray(cfg.fixed_lengths, dtype=np.int32)
    rng = np.random.default_rng([cfg.seed, 777])
    if cfg.uniform is not None:
        lo, hi = cfg.uniform
        return rng.integers(lo, hi + 1, size=cfg.batch).astype(np.int32)
    sigma = cfg.resp_sigma
    mu = math.log(cfg.resp_mean) - 0.5 * sigma * sigma
    resp = np.rint(np.exp(rng.normal(mu, sigma, size=cfg.batch)))
    resp = np.clip(resp, 1, cfg.resp_cap).astype(np.int64)
    return (cfg.prompt_len + resp).astype(np.int32)


def outlier_channels(cfg: Config) -> np.ndarray:
    rng = np.random.default_rng([cfg.seed, 999])
    return np.sort(rng.choice(cfg.head_dim, size=cfg.n_outlier, replace=False))


# ---------------------------------------------------------------- host data ---
def _kv_draw(rng, n, cfg: Config, outl):
    K = rng.standard_normal((n, cfg.num_kv_heads, cfg.head_dim), dtype=np.float32)
    K[:, :, outl] *= np.float32(8.0)
    V = rng.standard_normal((n, cfg.num_kv_heads, cfg.head_dim), dtype=np.float32)
    return K, V


def host_sequence(cfg: Config, layer: int, b: int, n_tokens: int):
    """bf16 bits: K, V [n_tokens][Hkv][D] and q [Hq][D] for sequence b."""
    rng = np.random.default_rng([cfg.seed, layer, b])
    K, V = _kv_draw(rng, n_tokens, cfg, outlier_channels(cfg))
    q = rng.standard_normal((cfg.num_q_heads, cfg.head_dim), dtype=np.float32)
    q *= np.float32(1.0 / math.sqrt(cfg.head_dim))
    return bf16_bits_from_f32(K), bf16_bits_from_f32(V), bf16_bits_from_f32(q)


def host_prompt(cfg: Config, layer: int, group: int):
    rng = np.random.default_rng([cfg.seed, layer, 10**6 + group])
    K, V = _kv_draw(rng, cfg.prompt_len, cfg, outlier_channels(cfg))
    return bf16_bits_from_f32(K), bf16_bits_from_f32(V)


def host_queries(cfg: Config, layer: int, batch: int, n_queries: int):
    """bf16 bits q [batch][n_queries][Hq][D] for multi-query decode."""
    rng = np.random.default_rng([cfg.seed, layer, 2 * 10**6 + n_queries])
    q = rng.standard_normal((batch, n_queries, cfg.num_q_heads, cfg.head_dim), dtype=np.float32)
    q *= np.float32(1.0 / math.sqrt(cfg.head_dim))
    return bf16_bits_from_f32(q)


# -------------------------------------------------------------- device data ---
def device_tokens(cfg: Config, layer: int, stream: int, n_tokens: int, device,
                  chunk: int = 1 << 20):
    """bf16 K, V tensors [n_tokens][Hkv][D] drawn on `device`."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(cfg.seed) * 1_000_003 + int(layer) * 10_007 + int(stream))
    outl = torch.as_tensor(outlier_channels(cfg), device=device)
    H, D = cfg.num_kv_heads, cfg.head_dim
    K = torch.empty((n_tokens, H, D), dtype=torch.bfloat16, device=device)
    V = torch.empty((n_tokens, H, D), dtype=torch.bfloat16, device=device)
    for s in range(0, n_tokens, chunk):
        e = min(n_tokens, s + chunk)
        k = torch.randn((e - s, H, D), generator=g, device=device, dtype=torch.float32)
        k[:, :, outl] *= 8.0
        K[s:e] = k.to(torch.bfloat16)
        V[s:e] = torch.randn((e - s, H, D), generator=g, device=device,
                             dtype=torch.float32).to(torch.bfloat16)
    return K, V


def device_queries(cfg: Config, layer: int, batch: int, device, n_queries: int = 0):
    """bf16 q [batch][Hq][D], or [batch][n_queries][Hq][D] when n_queries > 0."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(cfg.seed) * 1_000_003 + int(layer) * 10_007 + 999_983 + 7 * n_queries)
    shape = (batch, cfg.num_q_heads, cfg.head_dim) if n_queries <= 0 else \
        (batch, n_queries, cfg.num_q_heads, cfg.head_dim)
    q = torch.randn(shape, generator=g, device=device, dtype=torch.float32) / math.sqrt(cfg.head_dim)
    return q.to(torch.bfloat16)


# ------------------------------------------------------------- page tables ---
class PageAllocator:
    """Logical-to-physical page tables for a batch of sequences.

    Sequences in the same prompt group (b // group) share the physical pages
    that hold the prompt (prompt_len must then be a multiple of the page
    size); every other page is private.  Physical ids are a seeded
    permutation of [0, num_pages).  Unused table entries hold 0.
    """

    def __init__(self, lengths: Sequence[int], page_size: int = 16, prompt_len: int = 0,
                 group: int = 1, seed: int = 0, max_pages: Optional[int] = None,
                 extra_pages: int = 0):
        lengths = np.asarray(lengths, dtype=np.int64)
        self.page_size = page_size
        B = lengths.size
        need = (lengths + page_size - 1) // page_size
        self.max_pages = int(max_pages if max_pages is not None else max(1, need.max(initial=1)))
        shared = prompt_len // page_size if group > 1 else 0
        if group > 1:
            assert prompt_len % page_size == 0
        logical: List[List[int]] = []
        nxt = 0
        group_pages = {}
        for b in range(B):
            row = []
            gidx = b // group
            for i in range(int(need[b])):
                if i < shared:
                    key = (gidx, i)
                    if key not in group_pages:
                        group_pages[key] = nxt
                        nxt += 1
                    row.append(group_pages[key])
                else:
                    row.append(nxt)
                    nxt += 1
            logical.append(row)
        self.num_pages = nxt + extra_pages
        perm = np.random.default_rng([seed, 555]).permutation(self.num_pages).astype(np.int32)
        pt = np.zeros((B, self.max_pages), dtype=np.int32)
        for b, row in enumerate(logical):
            if row:
                pt[b, :len(row)] = perm[np.asarray(row)]
        self.page_table = pt
        self.shared_pages = shared
        self.unique_pages = nxt

    def pages_of(self, b: int, n_positions: int) -> np.ndarray:
        n = (n_positions + self.page_size - 1) // self.page_size
        return self.page_table[b, :n]
