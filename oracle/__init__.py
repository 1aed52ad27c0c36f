"""Float64 CPU oracle for paged grouped-query attention (ctypes wrapper).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. It shares no code
with the HIP library and never imports it.

The arithmetic lives in ``oracle.c`` (plain C, float64); this module only
marshals numpy arrays. Element storage is passed as raw bits: ``uint16``
for bf16 and ``uint8`` for OCP E4M3FN codes.

Cache layouts the oracle reads (its own, from the pages' description):
  * paged: ``[n_pages][Hkv][256][D]`` for K and for V, pages
    ``page_stride`` elements apart, position t in page ``PT[t // 256]``,
    slot ``t % 256`` (TensorFold pull request #2011, review section
    "Is paged output the same as windowed output?");
  * logical: ``[n_positions][Hkv][D]`` (no page table).
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from .build import LIB, build

PAGE_POSITIONS = 256
DTYPE_BF16 = 0
DTYPE_E4M3 = 1

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        lib = C.CDLL(LIB)
        P = C.c_void_p
        i32, i64, f32, f64 = C.c_int, C.c_int64, C.c_float, C.c_double
        lib.oracle_bf16_to_f64.restype = f64
        lib.oracle_bf16_to_f64.argtypes = [C.c_uint16]
        lib.oracle_e4m3_to_f64.restype = f64
        lib.oracle_e4m3_to_f64.argtypes = [C.c_uint8]
        lib.oracle_e4m3_encode.restype = C.c_uint8
        lib.oracle_e4m3_encode.argtypes = [f32, f32]
        lib.oracle_e4m3_encode_array.restype = None
        lib.oracle_e4m3_encode_array.argtypes = [P, i64, f32, P]
        lib.oracle_bf16_to_f64_array.restype = None
        lib.oracle_bf16_to_f64_array.argtypes = [P, i64, P]
        lib.oracle_e4m3_to_f64_array.restype = None
        lib.oracle_e4m3_to_f64_array.argtypes = [P, i64, P]
        lib.oracle_store.restype = i32
        lib.oracle_store.argtypes = [P, P, i32, f32, f32, P, i64, i32, i32, P, P, i64, i64, i32]
        lib.oracle_gather.restype = i32
        lib.oracle_gather.argtypes = [P, P, i32, f64, f64, P, i64, i32, i32, i64, P, P]
        lib.oracle_attention.restype = i32
        lib.oracle_attention.argtypes = [P, P, i32, f64, f64, P, i64, i32, i32, i64, P, i32, i64,
                                         P, P, i32, f64, P, i32]
        lib.oracle_attention_split.restype = i32
        lib.oracle_attention_split.argtypes = [P, P, i32, f64, f64, P, i64, i32, i32, i64, P, i32,
                                               i64, P, P, i32, f64, i64, i64, P, P, P, i32]
        lib.oracle_merge.restype = i32
        lib.oracle_merge.argtypes = [P, P, P, i64, i64, i32, P]
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


# ----------------------------------------------------------------------------- codecs

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    b = _c(bits, np.uint16)
    out = np.empty(b.shape, np.float64)
    _load().oracle_bf16_to_f64_array(_ptr(b), b.size, _ptr(out))
    return out


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """Exact value of OCP E4M3FN codes (uint8); 0x7F/0xFF are NaN."""
    b = _c(codes, np.uint8)
    out = np.empty(b.shape, np.float64)
    _load().oracle_e4m3_to_f64_array(_ptr(b), b.size, _ptr(out))
    return out


def e4m3_encode(x: np.ndarray, scale: float) -> np.ndarray:
    """Store quantiser: RNE(clamp(fl32(x / scale), +-448)) to E4M3FN codes."""
    a = _c(x, np.float32)
    out = np.empty(a.shape, np.uint8)
    _load().oracle_e4m3_encode_array(_ptr(a), a.size, float(np.float32(scale)), _ptr(out))
    return out


# ----------------------------------------------------------------------------- cache

def store(k_dst: np.ndarray, v_dst: np.ndarray, dtype: int, k_rows: np.ndarray,
          v_rows: np.ndarray, first_pos: int, page_table: np.ndarray | None = None,
          page_stride: int = 0, k_scale: float = 1.0, v_scale: float = 1.0,
          n_threads: int = 0) -> None:
    """Write rows ``[n][Hkv][D]`` (bf16 bits) at positions first_pos.. into the
    oracle-layout cache arrays ``k_dst``/``v_dst`` (modified in place)."""
    n, hkv, d = k_rows.shape
    kr, vr = _c(k_rows, np.uint16), _c(v_rows, np.uint16)
    pt = _c(page_table, np.int32)
    assert k_dst.flags.c_contiguous and v_dst.flags.c_contiguous
    rc = _load().oracle_store(_ptr(k_dst), _ptr(v_dst), dtype, float(k_scale), float(v_scale),
                              _ptr(pt), int(page_stride), hkv, d, _ptr(kr), _ptr(vr),
                              int(first_pos), n, int(n_threads))
    if rc != 0:
        raise ValueError(f"oracle_store failed ({rc})")


def gather(k_src, v_src, dtype, n_kv_heads, head_dim, n_keys, page_table=None, page_stride=0,
           k_scale=1.0, v_scale=1.0):
    """Logical float64 K, V ``[Hkv][n_keys][D]`` decoded from a cache."""
    pt = _c(page_table, np.int32)
    k = np.empty((n_kv_heads, n_keys, head_dim), np.float64)
    v = np.empty_like(k)
    _load().oracle_gather(_ptr(k_src), _ptr(v_src), dtype, float(k_scale), float(v_scale),
                          _ptr(pt), int(page_stride), n_kv_heads, head_dim, int(n_keys),
                          _ptr(k), _ptr(v))
    return k, v


def attention(k_src, v_src, dtype, q_bits, first_pos, n_kv_heads, n_keys_stored,
              page_table=None, page_stride=0, rows=None, sm_scale=None, k_scale=1.0,
              v_scale=1.0, n_threads=0, tree=None):
    """Float64 attention output ``[n_sel][Hq][D]`` for selected rows of one stream.

    q_bits: bf16 bits ``[n_rows][Hq][D]``; row i is at position first_pos + i
    and sees keys 0..first_pos+i.  ``rows`` selects row indices (default all).
    tree: optional ancestor words (uint32, one per row, at most 32 rows): row
    i then sees the keys before first_pos and the key first_pos + j (j <= i)
    only where bit j of its word is set.
    """
    q = _c(q_bits, np.uint16)
    n_rows, hq, d = q.shape
    sel = np.arange(n_rows, dtype=np.int32) if rows is None else _c(rows, np.int32)
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d)
    out = np.empty((len(sel), hq, d), np.float64)
    pt = _c(page_table, np.int32)
    tr = _c(tree, np.uint32)
    rc = _load().oracle_attention(_ptr(k_src), _ptr(v_src), dtype, float(k_scale),
                                  float(v_scale), _ptr(pt), int(page_stride), n_kv_heads, d,
                                  int(n_keys_stored), _ptr(q), hq, int(first_pos), _ptr(tr),
                                  _ptr(sel), len(sel), float(sm_scale), _ptr(out),
                                  int(n_threads))
    if rc != 0:
        raise ValueError(f"oracle_attention failed ({rc})")
    return out


def attention_split(k_src, v_src, dtype, q_bits, first_pos, n_kv_heads, n_keys_stored,
                    split_keys, n_split, page_table=None, page_stride=0, rows=None,
                    sm_scale=None, k_scale=1.0, v_scale=1.0, n_threads=0, tree=None):
    """Split-K form: (m, l, o) per (row, head, split) in float64."""
    q = _c(q_bits, np.uint16)
    n_rows, hq, d = q.shape
    sel = np.arange(n_rows, dtype=np.int32) if rows is None else _c(rows, np.int32)
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d)
    m = np.empty((len(sel), hq, n_split), np.float64)
    l = np.empty_like(m)
    o = np.empty((len(sel), hq, n_split, d), np.float64)
    pt = _c(page_table, np.int32)
    tr = _c(tree, np.uint32)
    rc = _load().oracle_attention_split(_ptr(k_src), _ptr(v_src), dtype, float(k_scale),
                                        float(v_scale), _ptr(pt), int(page_stride), n_kv_heads,
                                        d, int(n_keys_stored), _ptr(q), hq, int(first_pos),
                                        _ptr(tr), _ptr(sel), len(sel), float(sm_scale),
                                        int(split_keys),
                                        int(n_split), _ptr(m), _ptr(l), _ptr(o), int(n_threads))
    if rc != 0:
        raise ValueError(f"oracle_attention_split failed ({rc})")
    return m, l, o


def merge(m, l, o):
    """Fixed-order log-sum-exp merge of split triples; returns ``[..., D]``."""
    m = _c(m, np.float64)
    l = _c(l, np.float64)
    o = _c(o, np.float64)
    n_split, d = o.shape[-2], o.shape[-1]
    items = int(np.prod(m.shape[:-1]))
    out = np.empty(m.shape[:-1] + (d,), np.float64)
    rc = _load().oracle_merge(_ptr(m), _ptr(l), _ptr(o), items, n_split, d, _ptr(out))
    if rc != 0:
        raise ValueError("oracle_merge: an item has no visible key")
    return out


def normalised_error(got, ref) -> float:
    """max |got - ref| / max |ref| over the whole tensor."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))
