"""Test-side helpers: bit views and building the oracle's own cache arrays
from a seeded workload.  Nothing here runs on the GPU."""
from __future__ import annotations

import numpy as np
import torch

import oracle

PAGE = 256


def bits16(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (no rounding)."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def oracle_dtype(wl) -> int:
    return oracle.DTYPE_BF16 if wl.kv_dtype == "bf16" else oracle.DTYPE_E4M3


def oracle_pool(wl):
    """Build the oracle-layout pool [n_pages][Hkv][256][D] (K and V) holding
    every paged stream's rows and the filler pages, using oracle.store."""
    hkv, d = wl.n_kv_heads, wl.head_dim
    np_dtype = np.uint16 if wl.kv_dtype == "bf16" else np.uint8
    kp = np.zeros((wl.n_pages, hkv, PAGE, d), np_dtype)
    vp = np.zeros_like(kp)
    ps = hkv * PAGE * d
    dt = oracle_dtype(wl)
    for s, st in enumerate(wl.streams):
        if st.layout != "paged":
            continue
        oracle.store(kp, vp, dt, bits16(wl.k_rows[s]), bits16(wl.v_rows[s]), 0,
                     page_table=st.pages, page_stride=ps, k_scale=wl.k_scale,
                     v_scale=wl.v_scale)
    if wl.filler_k is not None and len(wl.filler_pages):
        oracle.store(kp, vp, dt, bits16(wl.filler_k), bits16(wl.filler_v), 0,
                     page_table=wl.filler_pages, page_stride=ps, k_scale=wl.k_scale,
                     v_scale=wl.v_scale)
    return kp, vp


def oracle_logical(wl, s):
    """The oracle-layout logical cache [ctx][Hkv][D] for stream s (any layout)."""
    st = wl.streams[s]
    np_dtype = np.uint16 if wl.kv_dtype == "bf16" else np.uint8
    k = np.zeros((st.ctx_len, wl.n_kv_heads, wl.head_dim), np_dtype)
    v = np.zeros_like(k)
    oracle.store(k, v, oracle_dtype(wl), bits16(wl.k_rows[s]), bits16(wl.v_rows[s]), 0,
                 k_scale=wl.k_scale, v_scale=wl.v_scale)
    return k, v


def oracle_reference(wl, s, rows=None, pool=None, n_threads=0):
    """Float64 oracle output [n_sel][Hq][D] for stream s of the workload."""
    st = wl.streams[s]
    q = bits16(wl.q[st.row_offset:st.row_offset + st.n_rows])
    dt = oracle_dtype(wl)
    if st.layout == "paged":
        kp, vp = pool if pool is not None else oracle_pool(wl)
        ps = wl.n_kv_heads * PAGE * wl.head_dim
        return oracle.attention(kp, vp, dt, q, st.first_pos, wl.n_kv_heads, st.ctx_len,
                                page_table=st.pages, page_stride=ps, rows=rows,
                                sm_scale=wl.sm_scale, k_scale=wl.k_scale, v_scale=wl.v_scale,
                                n_threads=n_threads, tree=st.tree)
    k, v = oracle_logical(wl, s)
    return oracle.attention(k, v, dt, q, st.first_pos, wl.n_kv_heads, st.ctx_len, rows=rows,
                            sm_scale=wl.sm_scale, k_scale=wl.k_scale, v_scale=wl.v_scale,
                            n_threads=n_threads, tree=st.tree)


def gpu_v_layout(v_rows: np.ndarray, vb: int) -> np.ndarray:
    """Rearrange V given as [..., positions, D] (positions a multiple of vb)
    into the device layout [..., positions/vb, D, vb]."""
    *lead, n, d = v_rows.shape
    x = v_rows.reshape(*lead, n // vb, vb, d)
    return np.swapaxes(x, -1, -2)
