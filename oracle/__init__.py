"""CPU oracle for KV4-RL decode attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never calls it and it
never calls the GPU library: the two share no code.  The arithmetic lives in
``kv4_oracle.c`` (plain C, fp64 after dequantization, fp32 quantizer
decisions); this module only builds it with gcc and marshals numpy arrays.
See ``kv4_oracle.h`` for the pages each function follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kv4_oracle.c")
# KV4_ORACLE_LIB loads another build of the same source (the sanitizer test's)
_LIB_PATH = os.environ.get("KV4_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

FMT_KV4, FMT_KV8, FMT_BF16 = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp",
               "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class Layout(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("group_size", ctypes.c_int32), ("n_sink", ctypes.c_int32),
                ("n_recent", ctypes.c_int32)]


def make_layout(hq, hkv, d, n_sink, n_recent, page=16, group=32) -> Layout:
    return Layout(hq, hkv, d, page, group, n_sink, n_recent)


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        L.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_bf16_to_f32.restype = ctypes.c_float
        L.orc_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.orc_f16_to_f64.restype = ctypes.c_double
        L.orc_f32_to_f16_rne.argtypes = [ctypes.c_float]
        L.orc_f32_to_f16_rne.restype = ctypes.c_uint16
        L.orc_quant_sym.argtypes = [P, ctypes.c_int, ctypes.c_int, P, P]
        L.orc_quant_sym.restype = None
        L.orc_block_bytes.argtypes = [ctypes.c_int, P]
        L.orc_block_bytes.restype = ctypes.c_size_t
        L.orc_side_bytes.argtypes = [P]
        L.orc_side_bytes.restype = ctypes.c_size_t
        L.orc_regions.argtypes = [ctypes.c_int] * 3 + [P] * 4
        L.orc_regions.restype = None
        L.orc_side_row.argtypes = [ctypes.c_int] * 3
        L.orc_side_row.restype = ctypes.c_int
        L.orc_append.argtypes = [ctypes.c_int, P, P, i64, P, i32, P, i32, P, P, i32, P, P, P]
        L.orc_append.restype = ctypes.c_int
        L.orc_gather.argtypes = [ctypes.c_int, P, P, i64, P, i32, P, i32, P, P, i32, i32, P, P, P]
        L.orc_gather.restype = ctypes.c_int
        L.orc_attend.argtypes = [ctypes.c_int, ctypes.c_int, P, P, P, P, ctypes.c_double, P, P, P]
        L.orc_attend.restype = None
        L.orc_probs.argtypes = [ctypes.c_int, ctypes.c_int, P, P, ctypes.c_double, P]
        L.orc_probs.restype = None
        L.orc_decode.argtypes = [ctypes.c_int, P, P, i64, P, i32, P, i32, P, P, i32, P,
                                 ctypes.c_double, P, i32, P, P, P, i32, i32]
        L.orc_decode.restype = ctypes.c_int
        L.orc_decode_mq.argtypes = [ctypes.c_int, P, P, i64, P, i32, P, i32, P, P, i32, P, i32,
                                    ctypes.c_double, P, i32, P, P, P, i32, i32]
        L.orc_decode_mq.restype = ctypes.c_int
        L.orc_cache_capacity.argtypes = [ctypes.c_int, P, i32, P, i32, ctypes.c_uint64, P, P]
        L.orc_cache_capacity.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return ctypes.c_void_p(a.ctypes.data)


# ---------------------------------------------------------------- scalars ---
def bf16_to_f32(bits: int) -> float:
    return float(lib().orc_bf16_to_f32(int(bits)))


def f16_to_f64(bits: int) -> float:
    return float(lib().orc_f16_to_f64(int(bits)))


def f32_to_f16(x: float) -> int:
    return int(lib().orc_f32_to_f16_rne(float(np.float32(x))))


def quant_sym(x_bf16: np.ndarray, qmax: int):
    """Quantize one group/row of bf16 bit patterns -> (int8 codes, fp16 bits)."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    codes = np.zeros(x.size, dtype=np.int8)
    s = np.zeros(1, dtype=np.uint16)
    lib().orc_quant_sym(_ptr(x), x.size, qmax, _ptr(codes), _ptr(s))
    return codes, int(s[0])


# ----------------------------------------------------------------- layout ---
def block_bytes(fmt: int, lay: Layout) -> int:
    return int(lib().orc_block_bytes(fmt, ctypes.byref(lay)))


def side_bytes(lay: Layout) -> int:
    return int(lib().orc_side_bytes(ctypes.byref(lay)))


def regions(n: int, S: int, R: int):
    out = np.zeros(4, dtype=np.int32)
    p = [ctypes.c_void_p(out.ctypes.data + 4 * i) for i in range(4)]
    lib().orc_regions(n, S, R, *p)
    se, mb, me, rb = (int(v) for v in out)
    return se, mb, me, rb


def side_row(p: int, S: int, R: int) -> int:
    return int(lib().orc_side_row(p, S, R))


# ---------------------------------------------------------- cache + decode ---
class HostCache:
    """Host byte arrays laid out exactly like the GPU pools."""

    def __init__(self, fmt, lay: Layout, num_pages: int, num_slots: int):
        self.fmt, self.lay = fmt, lay
        self.num_pages, self.num_slots = int(num_pages), int(num_slots)
        self.pages = np.zeros(num_pages * lay.num_kv_heads * block_bytes(fmt, lay), dtype=np.uint8)
        sb = side_bytes(lay) if fmt == FMT_KV4 else 0
        self.side = np.zeros(max(1, num_slots * lay.num_kv_heads * sb), dtype=np.uint8)


def append(cache: HostCache, page_table, seq_lens, slot_ids, k_new, v_new, cu_new):
    pt = np.ascontiguousarray(page_table, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    si = None if slot_ids is None else np.ascontiguousarray(slot_ids, dtype=np.int32)
    k = np.ascontiguousarray(k_new, dtype=np.uint16)
    v = np.ascontiguousarray(v_new, dtype=np.uint16)
    cu = np.ascontiguousarray(cu_new, dtype=np.int32)
    rc = lib().orc_append(cache.fmt, ctypes.byref(cache.lay), _ptr(cache.pages), cache.num_pages,
                          _ptr(cache.side), cache.num_slots, _ptr(pt), pt.shape[1], _ptr(sl),
                          _ptr(si), sl.size, _ptr(k), _ptr(v), _ptr(cu))
    if rc != 0:
        raise ValueError(f"oracle append rejected its input (code {rc})")


def gather(cache: HostCache, page_table, seq_lens, slot_ids, b: int, h: int):
    """Dequantized rows (fp64) the attention reads for (b, h), plus regions."""
    pt = np.ascontiguousarray(page_table, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    si = None if slot_ids is None else np.ascontiguousarray(slot_ids, dtype=np.int32)
    n = int(sl[b])
    D = cache.lay.head_dim
    K = np.zeros((max(n, 1), D), dtype=np.float64)
    V = np.zeros((max(n, 1), D), dtype=np.float64)
    reg = np.zeros(max(n, 1), dtype=np.uint8)
    rc = lib().orc_gather(cache.fmt, ctypes.byref(cache.lay), _ptr(cache.pages), cache.num_pages,
                          _ptr(cache.side), cache.num_slots, _ptr(pt), pt.shape[1], _ptr(sl),
                          _ptr(si), b, h, _ptr(K), _ptr(V), _ptr(reg))
    if rc < 0:
        raise ValueError(f"oracle gather rejected its input (code {rc})")
    return K[:n], V[:n], reg[:n]


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, region=None, sm_scale=1.0):
    q = np.ascontiguousarray(q, dtype=np.float64)
    K = np.ascontiguousarray(K, dtype=np.float64)
    V = np.ascontiguousarray(V, dtype=np.float64)
    n, D = K.shape
    reg = None if region is None else np.ascontiguousarray(region, dtype=np.uint8)
    out = np.zeros(D, dtype=np.float64)
    lse = np.zeros(1, dtype=np.float64)
    gap = np.zeros(1, dtype=np.float64)
    lib().orc_attend(n, D, _ptr(q), _ptr(K), _ptr(V), _ptr(reg), float(sm_scale),
                     _ptr(out), _ptr(lse), _ptr(gap))
    return out, float(lse[0]), float(gap[0])


def probs(q: np.ndarray, K: np.ndarray, sm_scale=1.0) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.float64)
    K = np.ascontiguousarray(K, dtype=np.float64)
    n, D = K.shape
    p = np.zeros(max(n, 1), dtype=np.float64)
    lib().orc_probs(n, D, _ptr(q), _ptr(K), float(sm_scale), _ptr(p))
    return p[:n]


def decode(cache: HostCache, page_table, seq_lens, slot_ids, q_bf16, sm_scale=1.0,
           subset=None, nthreads=0, q_int8=False):
    """Returns (out[n][Hq][D] fp64, lse[n][Hq] fp64, max merge gap).  q_int8:
    the integer-query variant (q quantized per query head, INT8 row rule)."""
    lay = cache.lay
    pt = np.ascontiguousarray(page_table, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    si = None if slot_ids is None else np.ascontiguousarray(slot_ids, dtype=np.int32)
    q = np.ascontiguousarray(q_bf16, dtype=np.uint16)
    sub = None if subset is None else np.ascontiguousarray(subset, dtype=np.int32)
    nseq = sl.size if sub is None else sub.size
    out = np.zeros((nseq, lay.num_q_heads, lay.head_dim), dtype=np.float64)
    lse = np.zeros((nseq, lay.num_q_heads), dtype=np.float64)
    gap = np.zeros(1, dtype=np.float64)
    rc = lib().orc_decode(cache.fmt, ctypes.byref(lay), _ptr(cache.pages), cache.num_pages,
                          _ptr(cache.side), cache.num_slots, _ptr(pt), pt.shape[1], _ptr(sl),
                          _ptr(si), sl.size, _ptr(q), float(sm_scale), _ptr(sub),
                          0 if sub is None else sub.size, _ptr(out), _ptr(lse), _ptr(gap),
                          int(nthreads), 1 if q_int8 else 0)
    if rc != 0:
        raise ValueError(f"oracle decode rejected its input (code {rc})")
    return out, lse, float(gap[0])


def decode_mq(cache: HostCache, page_table, seq_lens, slot_ids, q_bf16, num_queries: int,
              sm_scale=1.0, subset=None, nthreads=0, q_int8=False):
    """Multi-query decode: q_bf16 [B][T][Hq][D]; returns (out[n][T][Hq][D] fp64,
    lse[n][T][Hq] fp64, max merge gap).  Query t of sequence b sees the first
    seq_lens[b] - T + t + 1 positions of the cache as it stands.  q_int8: the
    integer-query variant, as in decode."""
    lay = cache.lay
    T = int(num_queries)
    pt = np.ascontiguousarray(page_table, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    si = None if slot_ids is None else np.ascontiguousarray(slot_ids, dtype=np.int32)
    q = np.ascontiguousarray(q_bf16, dtype=np.uint16)
    assert q.size == sl.size * T * lay.num_q_heads * lay.head_dim
    sub = None if subset is None else np.ascontiguousarray(subset, dtype=np.int32)
    nseq = sl.size if sub is None else sub.size
    out = np.zeros((nseq, T, lay.num_q_heads, lay.head_dim), dtype=np.float64)
    lse = np.zeros((nseq, T, lay.num_q_heads), dtype=np.float64)
    gap = np.zeros(1, dtype=np.float64)
    rc = lib().orc_decode_mq(cache.fmt, ctypes.byref(lay), _ptr(cache.pages), cache.num_pages,
                             _ptr(cache.side), cache.num_slots, _ptr(pt), pt.shape[1], _ptr(sl),
                             _ptr(si), sl.size, _ptr(q), T, float(sm_scale), _ptr(sub),
                             0 if sub is None else sub.size, _ptr(out), _ptr(lse), _ptr(gap),
                             int(nthreads), 1 if q_int8 else 0)
    if rc != 0:
        raise ValueError(f"oracle multi-query decode rejected its input (code {rc})")
    return out, lse, float(gap[0])


def cache_capacity(fmt: int, lay: Layout, num_layers: int, seq_lens, budget: int):
    """(bytes of all sequences, how many leading sequences fit in budget)."""
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    tot = np.zeros(1, dtype=np.uint64)
    fit = np.zeros(1, dtype=np.int32)
    rc = lib().orc_cache_capacity(fmt, ctypes.byref(lay), int(num_layers), _ptr(sl), sl.size,
                                  ctypes.c_uint64(int(budget)), _ptr(tot), _ptr(fit))
    if rc != 0:
        raise ValueError(f"oracle capacity rejected its input (code {rc})")
    return int(tot[0]), int(fit[0])
