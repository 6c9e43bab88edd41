"""Build a workload's cache on the GPU with libkv4's append.

Two builders:
  * build_from_host -- small cases: per-sequence numpy draws (workloads.gen
    host recipe), one bulk append.
  * build_config    -- the benchmark workloads: draws on the device, shared
    prompt pages appended once per group (the members' side blocks are then
    copied from the group leader, the way a prefix-sharing cache forks), then
    every response; the last position of each sequence is held back so the
    benchmark step can append it.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

import int4_kv_cache_amd as kv4
from workloads import (PageAllocator, context_lengths, get_config, host_prompt, host_sequence)
from workloads.gen import device_queries, device_tokens

ORACLE_FMT = {kv4.FMT_KV4: 0, kv4.FMT_KV8: 1, kv4.FMT_BF16: 2}


@dataclass
class GpuWorkload:
    cfg: object
    fmt: int
    layout: kv4.Layout
    cache: kv4.Cache
    alloc: PageAllocator
    lengths: np.ndarray              # context length at decode (includes the step token)
    batch: kv4.Batch                 # seq_lens = lengths (after the step append)
    q: object                        # bf16 [B][Hq][D]
    out: object
    lse: object
    workspace: object
    # the benchmark step's append (one token per sequence)
    step_k: Optional[object] = None
    step_v: Optional[object] = None
    step_cu: Optional[object] = None
    step_batch: Optional[kv4.Batch] = None
    # where every sequence's tokens are, to rebuild them on the host
    tokens: Dict[str, object] = field(default_factory=dict)

    # ---------------------------------------------------------------- ops --
    def step_append(self, stream=None):
        kv4.append(self.cache, self.step_batch, self.step_k, self.step_v, self.step_cu, stream)

    def decode(self, stream=None):
        kv4.decode(self.cache, self.batch, self.q, self.out, self.lse, self.workspace, 1.0, stream)

    def step_launches(self, stream=None):
        """The benchmark's decode step as its three launches, in stream order:
        the append of the step tokens with the plan in the same launch
        (kv4_append_decode_phases with PHASE_PLAN), then ATTEND, then MERGE.
        bench.py times exactly these calls; the parity tests run them too."""
        def plan():
            kv4.append_decode_phases(self.cache, self.step_batch, self.step_k, self.step_v, self.step_cu,
                                     self.q, self.out, self.lse, self.workspace, kv4.PHASE_PLAN, stream=stream)

        def attend():
            kv4.decode_phases(self.cache, self.batch, self.q, self.out, self.lse, self.workspace,
                              kv4.PHASE_ATTEND, stream=stream)

        def merge():
            kv4.decode_phases(self.cache, self.batch, self.q, self.out, self.lse, self.workspace,
                              kv4.PHASE_MERGE, stream=stream)

        return plan, attend, merge

    def plan_chunk_pages(self) -> int:
        """Middle pages per work item that the last plan chose (workspace header)."""
        import torch

        return int(self.workspace[:16].view(torch.int32).cpu()[2])

    # ------------------------------------------------------- host rebuild --
    def host_tokens(self, b: int):
        """bf16 bits K, V [L_b][Hkv][D] of sequence b, in position order."""
        t = self.tokens
        if "host_k" in t:
            return t["host_k"][b], t["host_v"][b]
        L = int(self.lengths[b])
        parts_k, parts_v = [], []
        if "prompt_k" in t:
            P = self.cfg.prompt_len
            g = b // self.cfg.group
            parts_k.append(t["prompt_k"][g * P:(g + 1) * P])
            parts_v.append(t["prompt_v"][g * P:(g + 1) * P])
        s, e = int(t["build_off"][b]), int(t["build_off"][b + 1])
        parts_k.append(t["build_k"][s:e])
        parts_v.append(t["build_v"][s:e])
        parts_k.append(self.step_k[b:b + 1])
        parts_v.append(self.step_v[b:b + 1])
        import torch

        K = torch.cat(parts_k).view(torch.int16).cpu().numpy().view(np.uint16)
        V = torch.cat(parts_v).view(torch.int16).cpu().numpy().view(np.uint16)
        assert K.shape[0] == L
        return K, V

    def host_q(self):
        import torch

        return self.q.view(torch.int16).cpu().numpy().view(np.uint16)


def _layout(cfg, fmt, n_sink=None, n_recent=None, int8_query=False):
    S = cfg.n_sink if n_sink is None else n_sink
    R = cfg.n_recent if n_recent is None else n_recent
    if fmt != kv4.FMT_KV4:
        S, R = 0, 0
        int8_query = False
    return kv4.make_layout(cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, S, R, int8_query=int8_query)


def _i32(a, device):
    import torch

    return torch.as_tensor(np.ascontiguousarray(a, dtype=np.int32), device=device)


def _bf16(a_bits, device):
    import torch

    return torch.as_tensor(np.ascontiguousarray(a_bits).view(np.int16), device=device).view(torch.bfloat16)


def _outputs(cfg, layout, B, max_pages, device):
    import torch

    out = torch.zeros((B, cfg.num_q_heads, cfg.head_dim), dtype=torch.bfloat16, device=device)
    lse = torch.zeros((B, cfg.num_q_heads), dtype=torch.float32, device=device)
    ws = torch.empty(kv4.workspace_bytes(layout, B, max_pages), dtype=torch.uint8, device=device)
    return out, lse, ws


def build_from_host(cfg_idx, fmt, lengths=None, n_sink=None, n_recent=None, device="cuda", int8_query=False,
                    token_by_token=False, slot_perm_seed=None, extra_pages=0, max_pages=None):
    """Small workloads: host draws per sequence, appended through the library."""
    import torch

    cfg = get_config(cfg_idx)
    lengths = np.asarray(context_lengths(cfg) if lengths is None else lengths, dtype=np.int32)
    B = lengths.size
    layout = _layout(cfg, fmt, n_sink, n_recent, int8_query)
    alloc = PageAllocator(lengths, seed=cfg.seed, extra_pages=extra_pages, max_pages=max_pages)
    cache = kv4.alloc_cache(fmt, layout, alloc.num_pages, B, device)
    hk, hv, hq = [], [], []
    for b in range(B):
        k, v, q = host_sequence(cfg, 0, b, int(lengths[b]))
        hk.append(k)
        hv.append(v)
        hq.append(q)
    slots = None
    if slot_perm_seed is not None:
        slots = np.random.default_rng(slot_perm_seed).permutation(B).astype(np.int32)
    pt = _i32(alloc.page_table, device)
    sl_t = _i32(slots, device) if slots is not None else None
    if token_by_token:
        for p in range(int(lengths.max(initial=0))):
            live = lengths > p
            n_new = live.astype(np.int32)
            sl = np.minimum(lengths, p + 1).astype(np.int32)
            cu = np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32)
            k = np.stack([hk[b][p] for b in range(B) if live[b]])
            v = np.stack([hv[b][p] for b in range(B) if live[b]])
            kv4.append(cache, kv4.Batch(pt, _i32(sl, device), sl_t), _bf16(k, device), _bf16(v, device),
                       _i32(cu, device))
    else:
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
        if cu[-1] > 0:
            k = np.concatenate(hk)
            v = np.concatenate(hv)
            kv4.append(cache, kv4.Batch(pt, _i32(lengths, device), sl_t), _bf16(k, device),
                       _bf16(v, device), _i32(cu, device))
    batch = kv4.Batch(pt, _i32(lengths, device), sl_t)
    q = _bf16(np.stack(hq), device)
    out, lse, ws = _outputs(cfg, layout, B, alloc.max_pages, device)
    wl = GpuWorkload(cfg, fmt, layout, cache, alloc, lengths, batch, q, out, lse, ws)
    wl.tokens = {"host_k": hk, "host_v": hv, "slots": slots}
    torch.cuda.synchronize()
    return wl


def build_config(cfg_idx, fmt, layer=0, n_sink=None, n_recent=None, device="cuda", int8_query=False,
                 keep_inputs=False, lengths=None):
    """Benchmark workloads: device draws; the last token of each sequence is
    left for the timed step (step_append)."""
    import torch

    cfg = get_config(cfg_idx)
    lengths = np.asarray(context_lengths(cfg) if lengths is None else lengths, dtype=np.int32)
    B = lengths.size
    layout = _layout(cfg, fmt, n_sink, n_recent, int8_query)
    shared = cfg.group > 1
    alloc = PageAllocator(lengths, prompt_len=cfg.prompt_len if shared else 0,
                          group=cfg.group, seed=cfg.seed)
    cache = kv4.alloc_cache(fmt, layout, alloc.num_pages, B, device)
    pt = _i32(alloc.page_table, device)
    P = cfg.prompt_len if shared else 0
    tokens = {}

    if shared:
        n_groups = (B + cfg.group - 1) // cfg.group
        pk, pv = device_tokens(cfg, layer, 1, n_groups * P, device)
        leaders = np.arange(0, B, cfg.group)
        lb = kv4.Batch(_i32(alloc.page_table[leaders], device), _i32(np.full(leaders.size, P), device),
                       _i32(leaders, device))
        cu = _i32(np.arange(leaders.size + 1) * P, device)
        kv4.append(cache, lb, pk, pv, cu)
        if cache.side is not None:
            sb = kv4.side_bytes(layout) * layout.num_kv_heads
            sv = cache.side.view(B, sb)
            src = torch.as_tensor((np.arange(B) // cfg.group) * cfg.group, device=device)
            sv.copy_(sv[src])
        tokens["prompt_k"], tokens["prompt_v"] = pk, pv

    n_build = (lengths - 1 - P).astype(np.int64)
    assert np.all(n_build >= 0)
    off = np.concatenate([[0], np.cumsum(n_build)])
    bk, bv = device_tokens(cfg, layer, 2, int(off[-1]), device)
    build_lens = (lengths - 1).astype(np.int32)
    if off[-1] > 0:
        kv4.append(cache, kv4.Batch(pt, _i32(build_lens, device)), bk, bv, _i32(off, device))
    tokens["build_off"] = off
    if keep_inputs:
        tokens["build_k"], tokens["build_v"] = bk, bv
    else:
        del bk, bv
        tokens.pop("prompt_k", None)
        tokens.pop("prompt_v", None)

    sk, sv_ = device_tokens(cfg, layer, 3, B, device)
    batch = kv4.Batch(pt, _i32(lengths, device))
    q = device_queries(cfg, layer, B, device)
    out, lse, ws = _outputs(cfg, layout, B, alloc.max_pages, device)
    wl = GpuWorkload(cfg, fmt, layout, cache, alloc, lengths, batch, q, out, lse, ws,
                     step_k=sk, step_v=sv_, step_cu=_i32(np.arange(B + 1), device), step_batch=batch)
    wl.tokens = tokens
    torch.cuda.synchronize()
    return wl


# ------------------------------------------------------------ many layers --
@dataclass
class LayerView:
    """One layer of a MultiLayerWorkload, with the attributes GpuWorkload has
    for the parity helpers (layout, cache, lengths, out, lse, host rebuild)."""
    parent: "MultiLayerWorkload"
    index: int

    def __getattr__(self, name):
        if name in ("cfg", "fmt", "layout", "alloc", "lengths", "batch", "workspace"):
            return getattr(self.parent, name)
        raise AttributeError(name)

    @property
    def cache(self):
        return self.parent.caches[self.index]

    @property
    def q(self):
        return self.parent.qs[self.index]

    @property
    def out(self):
        return self.parent.out[self.index]

    @property
    def lse(self):
        return self.parent.lse[self.index]

    @property
    def tokens(self):
        return {"slots": None}

    def host_tokens(self, b: int):
        return self.parent.host_tokens(self.index, b)

    def host_q(self):
        import torch

        return self.q.view(torch.int16).cpu().numpy().view(np.uint16)


@dataclass
class MultiLayerWorkload:
    """A decode step over many layers: one page table, seq_lens and plan for
    the batch; per layer its own cache (pages + side), q, out and lse."""
    cfg: object
    fmt: int
    layout: kv4.Layout
    alloc: PageAllocator
    lengths: np.ndarray
    batch: kv4.Batch
    caches: list
    qs: list
    out: object                      # bf16 [layers][B][Hq][D]
    lse: object                      # fp32 [layers][B][Hq]
    workspace: object
    chunks: np.ndarray               # sequence boundaries of the draw chunks
    _host: Dict = field(default_factory=dict)

    @property
    def n_layers(self) -> int:
        return len(self.caches)

    def layer(self, l: int) -> LayerView:
        return LayerView(self, l)

    def plan(self, stream=None):
        c = self.caches[0]
        kv4.decode_phases(c, self.batch, None, None, None, self.workspace, kv4.PHASE_PLAN,
                          stream=stream)

    def attend_layer(self, l: int, stream=None):
        kv4.decode_phases(self.caches[l], self.batch, self.qs[l], self.out[l], self.lse[l], self.workspace,
                          kv4.PHASE_ATTEND | kv4.PHASE_MERGE, stream=stream)

    def step(self, stream=None):
        """The decode of every layer: one plan, then attend + merge per layer."""
        self.plan(stream)
        for l in range(self.n_layers):
            self.attend_layer(l, stream)

    def _chunk_of(self, b: int) -> int:
        return int(np.searchsorted(self.chunks, b, side="right") - 1)

    def host_tokens(self, l: int, b: int):
        """bf16 bits K, V [L_b][Hkv][D] of sequence b in layer l, redrawn on the
        device from the chunk's seed (the draws are not kept)."""
        key = (l, b)
        if key not in self._host:
            c = self._chunk_of(b)
            s, e = int(self.chunks[c]), int(self.chunks[c + 1])
            off = np.concatenate([[0], np.cumsum(self.lengths[s:e].astype(np.int64))])
            k, v = device_tokens(self.cfg, l, 100 + c, int(off[-1]), self.caches[l].pages.device)
            import torch

            for bb in range(s, e):
                if (l, bb) in self._wanted or bb == b:
                    lo, hi = int(off[bb - s]), int(off[bb - s + 1])
                    self._host[(l, bb)] = (k[lo:hi].view(torch.int16).cpu().numpy().view(np.uint16),
                                           v[lo:hi].view(torch.int16).cpu().numpy().view(np.uint16))
            del k, v
        return self._host.pop(key)

    _wanted: set = field(default_factory=set)

    def want(self, l: int, sample):
        """Announce the sequences of layer l that host_tokens will be asked for,
        so one redraw of a chunk serves all of them."""
        for b in sample:
            self._wanted.add((l, int(b)))


def build_layers(cfg_idx, fmt, n_layers=None, device="cuda", chunk_seqs=32, n_sink=None, n_recent=None,
                 int8_query=False,
                 progress=None):
    """Many-layer workload: every layer's cache is built with device draws,
    chunk by chunk of sequences (so the bf16 draws of a whole layer are never
    resident at once); all L tokens of every sequence are appended."""
    import torch

    cfg = get_config(cfg_idx)
    L = int(cfg.layers if n_layers is None else n_layers)
    lengths = np.asarray(context_lengths(cfg), dtype=np.int32)
    B = lengths.size
    layout = _layout(cfg, fmt, n_sink, n_recent, int8_query)
    alloc = PageAllocator(lengths, seed=cfg.seed)
    pt = _i32(alloc.page_table, device)
    sl = _i32(lengths, device)
    chunks = np.arange(0, B + chunk_seqs, chunk_seqs)
    chunks[-1] = B
    chunks = np.unique(chunks)
    caches, qs = [], []
    for l in range(L):
        cache = kv4.alloc_cache(fmt, layout, alloc.num_pages, B, device)
        for c in range(len(chunks) - 1):
            s, e = int(chunks[c]), int(chunks[c + 1])
            off = np.concatenate([[0], np.cumsum(lengths[s:e].astype(np.int64))])
            k, v = device_tokens(cfg, l, 100 + c, int(off[-1]), device)
            bt = kv4.Batch(pt[s:e], sl[s:e], _i32(np.arange(s, e), device))
            kv4.append(cache, bt, k, v, _i32(off, device))
            del k, v
        caches.append(cache)
        qs.append(device_queries(cfg, l, B, device))
        torch.cuda.synchronize()
        if progress:
            progress(l)
    out = torch.zeros((L, B, cfg.num_q_heads, cfg.head_dim), dtype=torch.bfloat16, device=device)
    lse = torch.zeros((L, B, cfg.num_q_heads), dtype=torch.float32, device=device)
    ws = torch.empty(kv4.workspace_bytes(layout, B, alloc.max_pages), dtype=torch.uint8, device=device)
    return MultiLayerWorkload(cfg, fmt, layout, alloc, lengths, kv4.Batch(pt, sl), caches, qs, out, lse, ws,
                              chunks)
