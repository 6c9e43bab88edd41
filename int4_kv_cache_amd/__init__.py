"""Python binding of libkv4 (MI355X / gfx950 decode attention over a paged
INT4 KV cache with an INT8 sink/recent side cache).

This module only marshals arguments: every step of append and decode runs in
the HIP kernels of ``libkv4.so``.  PyTorch tensors provide device memory and
the current HIP stream.  Importing the package does not load the library;
``load()`` does, and raises if the shared library is missing -- there is no
fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
# KV4_LIB loads another build of the same sources (the host-sanitizer test's)
LIB_PATH = os.environ.get("KV4_LIB") or os.path.join(_HERE, "libkv4.so")

FMT_KV4, FMT_KV8, FMT_BF16 = 0, 1, 2
_PREFIX = {FMT_KV4: "kv4", FMT_KV8: "kv8", FMT_BF16: "kvbf16"}

STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported shape", -3: "workspace too small",
          -4: "kernel launch failed"}


class Kv4Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} returned {status} ({STATUS.get(status, 'unknown')})")
        self.status = status


class Layout(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("group_size", ctypes.c_int32), ("n_sink", ctypes.c_int32),
                ("n_recent", ctypes.c_int32), ("flags", ctypes.c_uint32)]


LAYOUT_WIDE_PROTECTION = 1  # lifts the n_sink + n_recent <= 144 bound to 4096
LAYOUT_INT8_QUERY = 2       # integer query-key products (kv4 decode only)


class CacheDesc(ctypes.Structure):
    _fields_ = [("pages", ctypes.c_void_p), ("num_pages", ctypes.c_int64),
                ("side", ctypes.c_void_p), ("num_slots", ctypes.c_int32)]


class BatchDesc(ctypes.Structure):
    _fields_ = [("page_table", ctypes.c_void_p), ("max_pages", ctypes.c_int32),
                ("seq_lens", ctypes.c_void_p), ("slot_ids", ctypes.c_void_p),
                ("batch", ctypes.c_int32)]


EXPORTS = [
    "kv4_abi_version", "kv4_status_string",
    "kv4_block_bytes", "kv8_block_bytes", "kvbf16_block_bytes", "kv4_side_bytes",
    "kv4_append", "kv8_append", "kvbf16_append",
    "kv4_decode_workspace_size",
    "kv4_decode_attention", "kv8_decode_attention", "kvbf16_decode_attention",
    "kv4_decode_phases", "kv8_decode_phases", "kvbf16_decode_phases",
    "kv4_decode_attention_mq", "kv8_decode_attention_mq", "kvbf16_decode_attention_mq",
    "kv4_append_decode_phases", "kv8_append_decode_phases", "kvbf16_append_decode_phases",
    "kv4_decode_attention_noalloc",
    "kv4_cache_capacity",
    "kv4_probe_blocks", "kv4_hbm_read_probe",
]

_lib = None


def load(path: Optional[str] = None):
    """Load libkv4.so and declare its signatures.  Raises if it is missing."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise FileNotFoundError(f"{p} not built: run `python -m int4_kv_cache_amd.build`")
    L = ctypes.CDLL(p)
    P, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    L.kv4_abi_version.restype = i32
    L.kv4_abi_version.argtypes = []
    L.kv4_status_string.restype = ctypes.c_char_p
    L.kv4_status_string.argtypes = [ctypes.c_int]
    for fn in ("kv4_block_bytes", "kv8_block_bytes", "kvbf16_block_bytes", "kv4_side_bytes"):
        getattr(L, fn).restype = sz
        getattr(L, fn).argtypes = [P]
    for pre in ("kv4", "kv8", "kvbf16"):
        f = getattr(L, f"{pre}_append")
        f.restype = ctypes.c_int
        f.argtypes = [P, P, P, P, P, P, i32, P]
        f = getattr(L, f"{pre}_decode_attention")
        f.restype = ctypes.c_int
        f.argtypes = [P, P, P, P, ctypes.c_float, P, P, P, sz, P]
        f = getattr(L, f"{pre}_decode_phases")
        f.restype = ctypes.c_int
        f.argtypes = [P, P, P, P, ctypes.c_float, P, P, P, sz, ctypes.c_uint32, P]
        f = getattr(L, f"{pre}_decode_attention_mq")
        f.restype = ctypes.c_int
        f.argtypes = [P, P, P, P, i32, ctypes.c_float, P, P, P, sz, P]
        f = getattr(L, f"{pre}_append_decode_phases")
        f.restype = ctypes.c_int
        f.argtypes = [P, P, P, P, P, P, i32, P, ctypes.c_float, P, P, P, sz, ctypes.c_uint32, P]
    L.kv4_decode_attention_noalloc.restype = ctypes.c_int
    L.kv4_decode_attention_noalloc.argtypes = [P, P, P, P, ctypes.c_float, P, P, P]
    L.kv4_decode_workspace_size.restype = ctypes.c_int
    L.kv4_decode_workspace_size.argtypes = [P, i32, i32, ctypes.POINTER(sz)]
    L.kv4_cache_capacity.restype = ctypes.c_int
    L.kv4_cache_capacity.argtypes = [P, i32, i32, P, i32, ctypes.c_uint64, ctypes.POINTER(ctypes.c_uint64),
                                     ctypes.POINTER(i32)]
    L.kv4_probe_blocks.restype = i32
    L.kv4_probe_blocks.argtypes = []
    L.kv4_hbm_read_probe.restype = ctypes.c_int
    L.kv4_hbm_read_probe.argtypes = [P, sz, P, P]
    if path is None:
        _lib = L
    return L


def _check(fn: str, status: int):
    if status != 0:
        raise Kv4Error(fn, status)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream=None) -> int:
    import torch

    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def make_layout(num_q_heads, num_kv_heads, head_dim, n_sink, n_recent, page_size=16,
                group_size=32, flags=None, int8_query=False) -> Layout:
    """flags None: KV4_LAYOUT_WIDE_PROTECTION exactly when n_sink + n_recent > 144,
    plus KV4_LAYOUT_INT8_QUERY when int8_query."""
    if flags is None:
        flags = LAYOUT_WIDE_PROTECTION if n_sink + n_recent > 144 else 0
        if int8_query:
            flags |= LAYOUT_INT8_QUERY
    return Layout(num_q_heads, num_kv_heads, head_dim, page_size, group_size, n_sink, n_recent, flags)


def block_bytes(fmt: int, layout: Layout) -> int:
    return int(getattr(load(), f"{_PREFIX[fmt]}_block_bytes")(ctypes.byref(layout)))


def side_bytes(layout: Layout) -> int:
    return int(load().kv4_side_bytes(ctypes.byref(layout)))


def workspace_bytes(layout: Layout, batch: int, max_pages: int) -> int:
    out = ctypes.c_size_t(0)
    _check("kv4_decode_workspace_size",
           load().kv4_decode_workspace_size(ctypes.byref(layout), batch, max_pages, ctypes.byref(out)))
    return int(out.value)


@dataclass
class Cache:
    """Device pools (uint8 torch tensors) in the library's layout."""
    fmt: int
    layout: Layout
    pages: "object"
    num_pages: int
    side: Optional["object"]
    num_slots: int

    def desc(self) -> CacheDesc:
        return CacheDesc(_ptr(self.pages), self.num_pages, _ptr(self.side), self.num_slots)


def alloc_cache(fmt: int, layout: Layout, num_pages: int, num_slots: int, device="cuda") -> Cache:
    import torch

    bb = block_bytes(fmt, layout)
    pages = torch.zeros(num_pages * layout.num_kv_heads * bb, dtype=torch.uint8, device=device)
    side = None
    if fmt == FMT_KV4 and layout.n_sink + layout.n_recent > 0:
        sb = side_bytes(layout)
        side = torch.zeros(num_slots * layout.num_kv_heads * sb, dtype=torch.uint8, device=device)
    return Cache(fmt, layout, pages, num_pages, side, num_slots if side is not None else 0)


@dataclass
class Batch:
    """Page table [B][max_pages], seq_lens [B], slot_ids [B] or None (int32, device)."""
    page_table: "object"
    seq_lens: "object"
    slot_ids: Optional["object"] = None

    def desc(self) -> BatchDesc:
        B, mp = self.page_table.shape
        return BatchDesc(_ptr(self.page_table), mp, _ptr(self.seq_lens), _ptr(self.slot_ids), B)


def append(cache: Cache, batch: Batch, k_new, v_new, cu_new, stream=None):
    """Quantize/store new tokens: k_new, v_new bf16 [T][Hkv][D]; cu_new int32 [B+1]."""
    T = int(k_new.shape[0])
    fn = f"{_PREFIX[cache.fmt]}_append"
    lay, cd, bd = cache.layout, cache.desc(), batch.desc()
    st = getattr(load(), fn)(ctypes.byref(lay), ctypes.byref(cd), ctypes.byref(bd), _ptr(k_new),
                             _ptr(v_new), _ptr(cu_new), T, _stream(stream))
    _check(fn, st)


def decode(cache: Cache, batch: Batch, q, out, lse, workspace, softmax_scale: float = 1.0,
           stream=None):
    """out bf16 [B][Hq][D], lse fp32 [B][Hq] (or None), workspace uint8 tensor."""
    fn = f"{_PREFIX[cache.fmt]}_decode_attention"
    lay, cd, bd = cache.layout, cache.desc(), batch.desc()
    st = getattr(load(), fn)(ctypes.byref(lay), ctypes.byref(cd), ctypes.byref(bd), _ptr(q),
                             float(softmax_scale), _ptr(out), _ptr(lse), _ptr(workspace),
                             int(workspace.numel()), _stream(stream))
    _check(fn, st)


NOALLOC_SCRATCH_BYTES = 64 << 20


def decode_noalloc(cache: Cache, batch: Batch, q, out, lse, softmax_scale: float = 1.0, stream=None):
    """kv4_decode_attention without a workspace: the library's fixed per-GPU
    scratch (NOALLOC_SCRATCH_BYTES) holds the plan and partials.  kv4 only."""
    if cache.fmt != FMT_KV4:
        raise ValueError("decode_noalloc exists for the kv4 format only")
    lay, cd, bd = cache.layout, cache.desc(), batch.desc()
    st = load().kv4_decode_attention_noalloc(ctypes.byref(lay), ctypes.byref(cd), ctypes.byref(bd), _ptr(q),
                                             float(softmax_scale), _ptr(out), _ptr(lse), _stream(stream))
    _check("kv4_decode_attention_noalloc", st)


MAX_QUERIES = 64


def cache_capacity(layout: Layout, fmt: int, num_layers: int, seq_lens, budget_bytes: int):
    """Host capacity model: (bytes of all sequences over num_layers layers,
    number of leading sequences that fit in budget_bytes).  seq_lens: host ints."""
    import numpy as np

    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    tot = ctypes.c_uint64(0)
    fit = ctypes.c_int32(0)
    st = load().kv4_cache_capacity(ctypes.byref(layout), int(fmt), int(num_layers),
                                   ctypes.c_void_p(sl.ctypes.data) if sl.size else None, int(sl.size),
                                   ctypes.c_uint64(int(budget_bytes)), ctypes.byref(tot), ctypes.byref(fit))
    _check("kv4_cache_capacity", st)
    return int(tot.value), int(fit.value)


def decode_mq(cache: Cache, batch: Batch, q, num_queries: int, out, lse, workspace,
              softmax_scale: float = 1.0, stream=None):
    """Multi-query decode: q/out bf16 [B][T][Hq][D], lse fp32 [B][T][Hq] (or None);
    query t of sequence b sees positions [0, seq_lens[b] - T + t + 1).  The
    workspace is workspace_size(layout, B * T, max_pages)."""
    fn = f"{_PREFIX[cache.fmt]}_decode_attention_mq"
    lay, cd, bd = cache.layout, cache.desc(), batch.desc()
    st = getattr(load(), fn)(ctypes.byref(lay), ctypes.byref(cd), ctypes.byref(bd), _ptr(q),
                             int(num_queries), float(softmax_scale), _ptr(out), _ptr(lse),
                             _ptr(workspace), int(workspace.numel()), _stream(stream))
    _check(fn, st)


PHASE_PLAN, PHASE_ATTEND, PHASE_MERGE = 1, 2, 4


def decode_phases(cache: Cache, batch: Batch, q, out, lse, workspace, phases: int,
                  softmax_scale: float = 1.0, stream=None):
    """The selected phases of a decode (PHASE_PLAN | PHASE_ATTEND | PHASE_MERGE);
    a plan in `workspace` serves later ATTEND/MERGE calls over the same batch."""
    fn = f"{_PREFIX[cache.fmt]}_decode_phases"
    lay, cd, bd = cache.layout, cache.desc(), batch.desc()
    st = getattr(load(), fn)(ctypes.byref(lay), ctypes.byref(cd), ctypes.byref(bd), _ptr(q),
                             float(softmax_scale), _ptr(out), _ptr(lse), _ptr(workspace),
                             int(workspace.numel()), int(phases), _stream(stream))
    _check(fn, st)


def append_decode_phases(cache: Cache, batch: Batch, k_new, v_new, cu_new, q, out, lse, workspace,
                         phases: int = PHASE_PLAN | PHASE_ATTEND | PHASE_MERGE, softmax_scale: float = 1.0,
                         stream=None):
    """append(...) then decode_phases(..., phases) in one call; with PHASE_PLAN
    the plan shares the append's launch."""
    fn = f"{_PREFIX[cache.fmt]}_append_decode_phases"
    T = int(k_new.shape[0]) if k_new is not None else 0
    lay, cd, bd = cache.layout, cache.desc(), batch.desc()
    st = getattr(load(), fn)(ctypes.byref(lay), ctypes.byref(cd), ctypes.byref(bd), _ptr(k_new), _ptr(v_new),
                             _ptr(cu_new), T, _ptr(q), float(softmax_scale), _ptr(out), _ptr(lse),
                             _ptr(workspace), int(workspace.numel()), int(phases), _stream(stream))
    _check(fn, st)


def hbm_read_probe(buf, sink, stream=None):
    _check("kv4_hbm_read_probe",
           load().kv4_hbm_read_probe(_ptr(buf), int(buf.numel() * buf.element_size()), _ptr(sink),
                                     _stream(stream)))


def probe_blocks() -> int:
    return int(load().kv4_probe_blocks())
