"""Host-side checks of the tensors behind a call, before anything launches.

The C ABI receives bare device pointers, so it cannot see how large, how
laid out or where a buffer is.  A short or strided tensor would turn into a
silent wrong result or an out-of-bounds device access (the stores write).
Every kernel entry point of the binding runs these checks first and raises
``ValueError`` on the first problem found; the C library then repeats its own
shape and range validation.

Every dtype, size and layout check of a call runs before any device check
(the device checks are collected in a list and run last by ``on_gpu``), so
each check can be exercised with host tensors in tests that have no GPU.
"""
from __future__ import annotations

import math

PAGE = 256


def _torch():
    import torch
    return torch


def kv_torch_dtype(kv_dtype: str):
    torch = _torch()
    if kv_dtype == "bf16":
        return torch.bfloat16
    if kv_dtype == "fp8":
        return torch.uint8
    raise ValueError(f"unknown KV dtype {kv_dtype!r} (expected 'bf16' or 'fp8')")


def extent_bytes(t) -> int:
    """Bytes addressable from t.data_ptr() to the end of its storage."""
    return t.untyped_storage().nbytes() - t.storage_offset() * t.element_size()


def on_gpu(dev: list) -> None:
    """The deferred device checks: every (name, tensor) must live on the GPU."""
    for name, t in dev:
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor (it is on {t.device})")


def _is_tensor(t) -> bool:
    return isinstance(t, _torch().Tensor)


def dense_rows(dev: list, name: str, t, heads: int | None, head_dim: int,
               min_rows: int) -> None:
    """A bf16 [rows][heads][head_dim] tensor, row-major, with >= min_rows rows."""
    torch = _torch()
    if not _is_tensor(t):
        raise ValueError(f"{name} must be a torch tensor")
    if t.dtype != torch.bfloat16:
        raise ValueError(f"{name} must be bfloat16, not {t.dtype}")
    if t.dim() != 3:
        raise ValueError(f"{name} must be [rows][heads][head_dim], got shape {tuple(t.shape)}")
    if t.shape[2] != head_dim:
        raise ValueError(f"{name}.shape[2] is {t.shape[2]}, the cache's head_dim is {head_dim}")
    if heads is not None and t.shape[1] != heads:
        raise ValueError(f"{name}.shape[1] is {t.shape[1]}, expected {heads}")
    if t.shape[0] < min_rows:
        raise ValueError(f"{name} has {t.shape[0]} rows; the streams use rows up to {min_rows}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    dev.append((name, t))


def _extent(name: str, t, dtype, elements: int) -> None:
    if not _is_tensor(t):
        raise ValueError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, not {t.dtype}")
    need = elements * t.element_size()
    if extent_bytes(t) < need:
        raise ValueError(f"{name} holds {extent_bytes(t)} bytes from its start, "
                         f"the call addresses {need}")


def cache(dev: list, c, need_pool: bool) -> None:
    """Pool tensors: the kernels address pages 0 .. n_pages-1, each
    n_kv_heads*256*head_dim elements at page_stride spacing (layer views are
    strided views into a larger pool, so the extent is what counts)."""
    dt = kv_torch_dtype(c.dtype)
    if c.head_dim <= 0 or c.n_kv_heads <= 0:
        raise ValueError("cache head_dim and n_kv_heads must be positive")
    if not need_pool:
        return
    if c.k_pages is None or c.v_pages is None:
        raise ValueError("a paged stream needs the cache's k_pages and v_pages")
    block = c.n_kv_heads * PAGE * c.head_dim
    ps = c.page_stride or block
    if c.n_pages < 1:
        raise ValueError("cache n_pages must be >= 1")
    elems = (c.n_pages - 1) * ps + block
    _extent("cache.k_pages", c.k_pages, dt, elems)
    _extent("cache.v_pages", c.v_pages, dt, elems)
    dev += [("cache.k_pages", c.k_pages), ("cache.v_pages", c.v_pages)]


def streams(dev: list, c, ss, max_rows: int | None = None) -> int:
    """Per-stream tensors of Stream descriptors (raw pa_stream structs are
    passed through unchecked).  Returns the rows the streams use in q / out /
    k_new: max(row_offset + n_rows)."""
    torch = _torch()
    from . import PA_LAYOUT_PAGED, PA_LAYOUT_SLAB, Stream
    dt = kv_torch_dtype(c.dtype)
    rows = 0
    for i, s in enumerate(ss):
        if not isinstance(s, Stream):
            continue
        if s.n_rows <= 0:
            continue
        if max_rows is not None and s.n_rows > max_rows:
            raise ValueError(f"stream {i}: {s.n_rows} rows, at most {max_rows} per call")
        rows = max(rows, int(s.row_offset) + int(s.n_rows))
        if s.layout == PA_LAYOUT_PAGED:
            pt = s.page_table
            if not _is_tensor(pt):
                raise ValueError(f"stream {i}: a paged stream needs a page_table tensor")
            if pt.dtype != torch.int32:
                raise ValueError(f"stream {i}: page_table must be int32, not {pt.dtype}")
            need = math.ceil(int(s.ctx_len) / PAGE)
            if pt.numel() < need:
                raise ValueError(f"stream {i}: page_table has {pt.numel()} ids, "
                                 f"context {s.ctx_len} needs {need}")
            if not pt.is_contiguous():
                raise ValueError(f"stream {i}: page_table must be contiguous")
            dev.append((f"stream {i} page_table", pt))
        elif s.layout == PA_LAYOUT_SLAB:
            elems = c.n_kv_heads * int(s.slab_cap) * c.head_dim
            _extent(f"stream {i} k_slab", s.k_slab, dt, elems)
            _extent(f"stream {i} v_slab", s.v_slab, dt, elems)
            dev += [(f"stream {i} k_slab", s.k_slab), (f"stream {i} v_slab", s.v_slab)]
        else:
            raise ValueError(f"stream {i}: unknown layout {s.layout}")
        tm = s.tree_mask
        if tm is not None:
            if not _is_tensor(tm) or tm.dtype != torch.int32:
                raise ValueError(f"stream {i}: tree_mask must be an int32 tensor")
            if tm.numel() < s.n_rows:
                raise ValueError(f"stream {i}: tree_mask has {tm.numel()} words for "
                                 f"{s.n_rows} rows")
            if not tm.is_contiguous():
                raise ValueError(f"stream {i}: tree_mask must be contiguous")
            dev.append((f"stream {i} tree_mask", tm))
    return rows


def any_paged(ss) -> bool:
    from . import PA_LAYOUT_PAGED, Stream
    return any(isinstance(s, Stream) and s.layout == PA_LAYOUT_PAGED and s.n_rows > 0
               for s in ss)


def workspace(dev: list, ws, need_bytes: int) -> None:
    if not _is_tensor(ws):
        raise ValueError("workspace must be a torch tensor")
    nb = ws.numel() * ws.element_size()
    if nb < need_bytes:
        raise ValueError(f"workspace holds {nb} bytes, the call needs {need_bytes}")
    if not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")
    dev.append(("workspace", ws))


def host_pages(name: str, t, n_bytes: int) -> None:
    if not _is_tensor(t):
        raise ValueError(f"{name} must be a torch tensor")
    if extent_bytes(t) < n_bytes:
        raise ValueError(f"{name} holds {extent_bytes(t)} bytes, the pages need {n_bytes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.is_cuda:
        raise ValueError(f"{name} must be host memory")
