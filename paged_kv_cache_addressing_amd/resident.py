"""Materialise a synthetic workload in device memory through ``write_kv``.

The pool, slabs, page tables and query rows are torch device tensors; every
KV byte is written by the library's own store kernel, so what the attention
kernels read is exactly what a serving engine would have stored.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import (PA_LAYOUT_PAGED, PA_LAYOUT_SLAB, PAGE_POSITIONS, KVCache, Stream, alloc_pool,
               alloc_slab, write_kv)


@dataclass
class Resident:
    cache: KVCache
    streams: list          # attention Stream descriptors (device pointers inside)
    q: torch.Tensor        # bf16 [rows][Hq][D] on device
    page_tables: list      # device int32 tensors (None for slabs)
    slabs: list            # (k, v) device tensors or None
    n_q_heads: int
    sm_scale: float
    split_keys: int


def _store(cache, descs, rows_k, rows_v, device):
    """One write_kv call storing whole-context rows for several targets."""
    if not descs:
        return
    k = torch.cat(rows_k).to(device)
    v = torch.cat(rows_v).to(device)
    write_kv(cache, descs, k, v)
    del k, v


def _tree(st, device):
    """The stream's ancestor words as a device int32 tensor, or None."""
    if getattr(st, "tree", None) is None:
        return None
    return torch.from_numpy(st.tree.view(np.int32).copy()).to(device)


def upload(wl, device: str = "cuda", poison_tail: bool = False,
           zero_pool: bool = True) -> Resident:
    """Upload workload ``wl`` (see the workloads module) and store its rows.

    poison_tail: fill never-written slots of each paged stream's last page
    with NaN bit patterns (bf16 0x7FC0, fp8 0x7F) before storing, so reads
    past a stream's length would show up as NaN.
    """
    hkv, d = wl.n_kv_heads, wl.head_dim
    cache = alloc_pool(max(wl.n_pages, 1), hkv, d, wl.kv_dtype, device, zero=zero_pool)
    cache.k_scale, cache.v_scale = wl.k_scale, wl.v_scale
    streams, tables, slabs = [], [], []
    store_descs, rk, rv = [], [], []
    at = 0
    for s, st in enumerate(wl.streams):
        if st.layout == "paged":
            pt = torch.from_numpy(st.pages).to(device=device, dtype=torch.int32)
            tables.append(pt)
            slabs.append(None)
            if poison_tail and st.ctx_len % PAGE_POSITIONS:
                last = int(st.pages[-1])
                j0 = st.ctx_len % PAGE_POSITIONS
                if wl.kv_dtype == "bf16":
                    nan = torch.tensor(0x7FC0, dtype=torch.int16).view(torch.bfloat16)
                else:
                    nan = torch.tensor(0x7F, dtype=torch.uint8)
                nan = nan.to(device)
                cache.k_pages[last, :, j0:, :] = nan
                vb = cache.v_pages.shape[-1]
                for b in range(PAGE_POSITIONS // vb):
                    start = max(j0 - b * vb, 0)
                    if start < vb:
                        cache.v_pages[last, :, b, :, start:] = nan
            desc = Stream(st.ctx_len, st.ctx_len, at, 0, page_table=pt, layout=PA_LAYOUT_PAGED)
            att = Stream(st.ctx_len, st.n_rows, st.row_offset, st.first_pos, page_table=pt,
                         layout=PA_LAYOUT_PAGED, tree_mask=_tree(st, device))
        else:
            ks, vs = alloc_slab(st.slab_cap, hkv, d, wl.kv_dtype, device, zero=True)
            tables.append(None)
            slabs.append((ks, vs))
            desc = Stream(st.ctx_len, st.ctx_len, at, 0, k_slab=ks, v_slab=vs,
                          slab_cap=st.slab_cap, layout=PA_LAYOUT_SLAB)
            att = Stream(st.ctx_len, st.n_rows, st.row_offset, st.first_pos, k_slab=ks, v_slab=vs,
                         slab_cap=st.slab_cap, layout=PA_LAYOUT_SLAB,
                         tree_mask=_tree(st, device))
        store_descs.append(desc)
        rk.append(wl.k_rows[s])
        rv.append(wl.v_rows[s])
        at += st.ctx_len
        streams.append(att)
        # keep host memory bounded for the large workloads: flush every ~256M elements
        if at * hkv * d >= (1 << 28):
            _store(cache, store_descs, rk, rv, device)
            store_descs, rk, rv, at = [], [], [], 0
    _store(cache, store_descs, rk, rv, device)
    if wl.filler_k is not None and len(wl.filler_pages):
        pt = torch.from_numpy(wl.filler_pages).to(device=device, dtype=torch.int32)
        n = len(wl.filler_pages) * PAGE_POSITIONS
        write_kv(cache, [Stream(n, n, 0, 0, page_table=pt)], wl.filler_k.to(device),
                 wl.filler_v.to(device))
    q = wl.q.to(device)
    torch.cuda.synchronize()
    return Resident(cache, streams, q, tables, slabs, wl.n_q_heads, wl.sm_scale, wl.split_keys)
