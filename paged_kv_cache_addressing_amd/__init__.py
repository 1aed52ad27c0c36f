"""Python binding of the gfx950 paged grouped-query attention library.

Argument marshalling only: every step of the hot path runs in the HIP
kernels of ``libpaged_attn.so`` (see ``include/paged_attn.h``).  PyTorch
provides device memory and streams.  There is no fallback: if the shared
library is missing, every compute call raises.

Entry points carry the C names: ``page_pool_create`` / ``page_pool_alloc`` /
``page_pool_free`` / ``page_pool_destroy`` / ``page_pool_free_count``,
``write_kv``, ``paged_attn_decode_workspace_size``, ``paged_attn_decode``,
``paged_attn_decode_plan``, ``paged_attn_prefill``, ``pa_status_string``.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

import numpy as np

from . import validate as _v

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpaged_attn.so")

PAGE_POSITIONS = 256
DEFAULT_SPLIT_KEYS = 4096
DECODE_MAX_ROWS = 16
TREE_MAX_ROWS = 32  # rows of a stream that carries an ancestor table
NOALLOC_SCRATCH_BYTES = 128 << 20  # the fixed scratch of paged_attn_decode_noalloc

PA_OK, PA_EINVAL, PA_ERANGE, PA_ENOSPC, PA_ETOOBIG, PA_EWORKSPACE, PA_EDEVICE, PA_EUNSUPPORTED = (
    0, -1, -2, -3, -4, -5, -6, -7)
PA_KV_BF16, PA_KV_FP8_E4M3 = 0, 1
PA_LAYOUT_PAGED, PA_LAYOUT_SLAB = 0, 1

EXPORTS = ["pa_status_string", "pa_version", "page_pool_create", "page_pool_destroy",
           "page_pool_alloc", "page_pool_free", "page_pool_free_count", "page_pool_share",
           "page_pool_refcount", "page_copy", "page_save", "page_restore", "write_kv",
           "paged_attn_decode_workspace_size", "paged_attn_decode", "paged_attn_decode_partials",
           "paged_attn_decode_merge", "paged_attn_decode_plan", "paged_attn_prefill",
           "paged_attn_decode_noalloc", "pa_hbm_read_probe"]


class PagedAttnError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


class pa_kv_cache(C.Structure):
    _fields_ = [("k_pages", C.c_void_p), ("v_pages", C.c_void_p), ("page_stride", C.c_int64),
                ("n_pages", C.c_int32), ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("dtype", C.c_int32), ("k_scale", C.c_float), ("v_scale", C.c_float)]


class pa_stream(C.Structure):
    _fields_ = [("layout", C.c_int32), ("ctx_len", C.c_int32), ("n_rows", C.c_int32),
                ("row_offset", C.c_int32), ("first_pos", C.c_int32), ("reserved", C.c_int32),
                ("page_table", C.c_void_p), ("k_slab", C.c_void_p), ("v_slab", C.c_void_p),
                ("slab_cap", C.c_int64), ("tree_mask", C.c_void_p)]


class pa_decode_plan(C.Structure):
    _fields_ = [("n_launch_groups", C.c_int32), ("total_splits", C.c_int32),
                ("col_tiles", C.c_int32), ("partial_blocks", C.c_int32),
                ("merge_blocks", C.c_int32), ("wide_blocks", C.c_int32),
                ("narrow_splits_per_wg", C.c_int32), ("workspace_bytes", C.c_size_t)]


_lib = None


def lib():
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                               "(run __graft_entry__.build())")
        L = C.CDLL(LIB_PATH)
        P, i32, i64, f32, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_float, C.c_size_t
        L.pa_status_string.restype = C.c_char_p
        L.pa_status_string.argtypes = [C.c_int]
        L.pa_version.restype = C.c_int
        L.pa_version.argtypes = []
        L.page_pool_create.restype = C.c_int
        L.page_pool_create.argtypes = [i32, C.POINTER(P)]
        L.page_pool_destroy.restype = None
        L.page_pool_destroy.argtypes = [P]
        L.page_pool_alloc.restype = C.c_int
        L.page_pool_alloc.argtypes = [P, i32, P]
        L.page_pool_free.restype = C.c_int
        L.page_pool_free.argtypes = [P, P, i32]
        L.page_pool_free_count.restype = i32
        L.page_pool_free_count.argtypes = [P]
        L.page_pool_share.restype = C.c_int
        L.page_pool_share.argtypes = [P, P, i32]
        L.page_pool_refcount.restype = i32
        L.page_pool_refcount.argtypes = [P, i32]
        L.page_copy.restype = C.c_int
        L.page_copy.argtypes = [C.POINTER(pa_kv_cache), P, P, i32, P]
        L.page_save.restype = C.c_int
        L.page_save.argtypes = [C.POINTER(pa_kv_cache), P, i32, P, P, P]
        L.page_restore.restype = C.c_int
        L.page_restore.argtypes = [C.POINTER(pa_kv_cache), P, i32, P, P, P]
        L.write_kv.restype = C.c_int
        L.write_kv.argtypes = [C.POINTER(pa_kv_cache), C.POINTER(pa_stream), i32, P, P, P]
        L.paged_attn_decode_workspace_size.restype = sz
        L.paged_attn_decode_workspace_size.argtypes = [C.POINTER(pa_stream), i32, i32, i32, i32]
        L.paged_attn_decode.restype = C.c_int
        L.paged_attn_decode.argtypes = [C.POINTER(pa_kv_cache), C.POINTER(pa_stream), i32, P, P,
                                        i32, f32, i32, P, sz, P]
        L.paged_attn_decode_partials.restype = C.c_int
        L.paged_attn_decode_partials.argtypes = [C.POINTER(pa_kv_cache), C.POINTER(pa_stream),
                                                 i32, P, i32, f32, i32, P, sz, P]
        L.paged_attn_decode_merge.restype = C.c_int
        L.paged_attn_decode_merge.argtypes = [C.POINTER(pa_kv_cache), C.POINTER(pa_stream), i32,
                                              P, i32, i32, P, sz, P]
        L.paged_attn_decode_plan.restype = C.c_int
        L.paged_attn_decode_plan.argtypes = [C.POINTER(pa_stream), i32, i32, i32, i32, i32, i32,
                                             P, C.POINTER(pa_decode_plan)]
        L.paged_attn_decode_noalloc.restype = C.c_int
        L.paged_attn_decode_noalloc.argtypes = [C.POINTER(pa_kv_cache), C.POINTER(pa_stream),
                                                i32, P, P, i32, f32, i32, P]
        L.pa_hbm_read_probe.restype = C.c_int
        L.pa_hbm_read_probe.argtypes = [P, sz, P, P]
        L.paged_attn_prefill.restype = C.c_int
        L.paged_attn_prefill.argtypes = [C.POINTER(pa_kv_cache), C.POINTER(pa_stream), i32, P, P,
                                         i32, f32, P]
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().pa_status_string(int(status)).decode()


pa_status_string = status_string


def _check(rc: int, what: str):
    if rc != PA_OK:
        raise PagedAttnError(rc, what)


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _hip_stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


# ----------------------------------------------------------------------------- descriptors

@dataclass
class KVCache:
    """Device pool tensors plus geometry; see pa_kv_cache in paged_attn.h.

    K page layout [n_pages][Hkv][256][D]; V page layout
    [n_pages][Hkv][256/VB][D][VB] with VB = 64 bytes of keys (see v_block).
    dtype: "bf16" (torch.bfloat16 storage) or "fp8" (uint8 E4M3FN codes).
    """
    k_pages: object
    v_pages: object
    n_pages: int
    n_kv_heads: int
    head_dim: int
    dtype: str = "bf16"
    k_scale: float = 1.0
    v_scale: float = 1.0
    page_stride: int | None = None

    def c(self) -> pa_kv_cache:
        ps = self.page_stride or self.n_kv_heads * PAGE_POSITIONS * self.head_dim
        return pa_kv_cache(_ptr(self.k_pages), _ptr(self.v_pages), ps, self.n_pages,
                           self.n_kv_heads, self.head_dim,
                           PA_KV_BF16 if self.dtype == "bf16" else PA_KV_FP8_E4M3,
                           float(self.k_scale), float(self.v_scale))


@dataclass
class Stream:
    """One stream of a call; see pa_stream in paged_attn.h."""
    ctx_len: int
    n_rows: int
    row_offset: int
    first_pos: int
    page_table: object = None     # torch.int32 device tensor (paged)
    k_slab: object = None         # device tensor [Hkv][cap][D]
    v_slab: object = None         # device tensor [Hkv][cap/VB][D][VB]
    slab_cap: int = 0
    layout: int = PA_LAYOUT_PAGED
    tree_mask: object = None      # int32 device tensor, one ancestor word per row

    def c(self) -> pa_stream:
        return pa_stream(int(self.layout), int(self.ctx_len), int(self.n_rows),
                         int(self.row_offset), int(self.first_pos), 0, _ptr(self.page_table),
                         _ptr(self.k_slab), _ptr(self.v_slab), int(self.slab_cap),
                         _ptr(self.tree_mask))


def _streams(streams):
    arr = (pa_stream * max(len(streams), 1))()
    for i, s in enumerate(streams):
        arr[i] = s.c() if isinstance(s, Stream) else s
    return arr, len(streams)


def v_block(dtype: str) -> int:
    """Keys per V block (64 bytes of one dim): 32 for bf16, 64 for fp8."""
    return 32 if dtype == "bf16" else 64


def alloc_pool(n_pages: int, n_kv_heads: int, head_dim: int, dtype: str = "bf16",
               device="cuda", zero: bool = True) -> KVCache:
    """Allocate pool tensors on the device (torch memory, caller-owned).

    K: [n_pages][Hkv][256][D]; V: [n_pages][Hkv][256/VB][D][VB] (see v_block).
    """
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.uint8
    vb = v_block(dtype)
    mk = torch.zeros if zero else torch.empty
    k = mk((n_pages, n_kv_heads, PAGE_POSITIONS, head_dim), dtype=tdt, device=device)
    v = mk((n_pages, n_kv_heads, PAGE_POSITIONS // vb, head_dim, vb), dtype=tdt, device=device)
    return KVCache(k, v, n_pages, n_kv_heads, head_dim, dtype)


def alloc_slab(cap: int, n_kv_heads: int, head_dim: int, dtype: str = "bf16", device="cuda",
               zero: bool = True):
    """Slab tensors K [Hkv][cap][D] and V [Hkv][cap/VB][D][VB]; cap a multiple of 256."""
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.uint8
    vb = v_block(dtype)
    mk = torch.zeros if zero else torch.empty
    return (mk((n_kv_heads, cap, head_dim), dtype=tdt, device=device),
            mk((n_kv_heads, cap // vb, head_dim, vb), dtype=tdt, device=device))


# ----------------------------------------------------------------------------- page pool

class PagePool:
    """Host bookkeeping of free page ids (page_pool_* in paged_attn.h)."""

    def __init__(self, n_pages: int):
        h = C.c_void_p()
        _check(lib().page_pool_create(int(n_pages), C.byref(h)), "page_pool_create")
        self._h = h
        self.n_pages = n_pages

    def alloc(self, n: int) -> np.ndarray:
        ids = np.empty(max(n, 1), np.int32)
        _check(lib().page_pool_alloc(self._h, int(n), ids.ctypes.data_as(C.c_void_p)),
               "page_pool_alloc")
        return ids[:n]

    def free(self, ids) -> None:
        a = np.ascontiguousarray(ids, np.int32)
        _check(lib().page_pool_free(self._h, a.ctypes.data_as(C.c_void_p), len(a)),
               "page_pool_free")

    def free_count(self) -> int:
        return int(lib().page_pool_free_count(self._h))

    def share(self, ids) -> None:
        """One more reference per occurrence of each id (a shared prefix page)."""
        a = np.ascontiguousarray(ids, np.int32)
        _check(lib().page_pool_share(self._h, a.ctypes.data_as(C.c_void_p), len(a)),
               "page_pool_share")

    def refcount(self, page: int) -> int:
        r = int(lib().page_pool_refcount(self._h, int(page)))
        if r < 0:
            raise PagedAttnError(r, "page_pool_refcount")
        return r

    def close(self):
        if self._h:
            lib().page_pool_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _ids(ids):
    return np.ascontiguousarray(ids, np.int32)


def _page_bytes(cache: KVCache) -> int:
    ps = cache.page_stride or cache.n_kv_heads * PAGE_POSITIONS * cache.head_dim
    return ps * (2 if cache.dtype == "bf16" else 1)


def page_copy(cache: KVCache, src_ids, dst_ids, stream=None) -> None:
    """Device copy of whole pages src_ids[i] -> dst_ids[i] (K and V)."""
    s, d = _ids(src_ids), _ids(dst_ids)
    if len(s) != len(d):
        raise ValueError("src_ids and dst_ids differ in length")
    dev = []
    _v.cache(dev, cache, len(s) > 0)
    _v.on_gpu(dev)
    cc = cache.c()
    _check(lib().page_copy(C.byref(cc), s.ctypes.data_as(C.c_void_p), d.ctypes.data_as(C.c_void_p),
                           len(s), _hip_stream(stream)), "page_copy")


def page_save(cache: KVCache, ids, host_k, host_v, stream=None) -> None:
    """Copy whole pages to host tensors (page ids[i] at row i of each)."""
    a = _ids(ids)
    dev = []
    _v.cache(dev, cache, len(a) > 0)
    if len(a):
        _v.host_pages("host_k", host_k, len(a) * _page_bytes(cache))
        _v.host_pages("host_v", host_v, len(a) * _page_bytes(cache))
    _v.on_gpu(dev)
    cc = cache.c()
    _check(lib().page_save(C.byref(cc), a.ctypes.data_as(C.c_void_p), len(a), _ptr(host_k),
                           _ptr(host_v), _hip_stream(stream)), "page_save")


def page_restore(cache: KVCache, ids, host_k, host_v, stream=None) -> None:
    """Copy host tensors (row i -> page ids[i]) back into the pool."""
    a = _ids(ids)
    dev = []
    _v.cache(dev, cache, len(a) > 0)
    if len(a):
        _v.host_pages("host_k", host_k, len(a) * _page_bytes(cache))
        _v.host_pages("host_v", host_v, len(a) * _page_bytes(cache))
    _v.on_gpu(dev)
    cc = cache.c()
    _check(lib().page_restore(C.byref(cc), a.ctypes.data_as(C.c_void_p), len(a), _ptr(host_k),
                              _ptr(host_v), _hip_stream(stream)), "page_restore")


def page_pool_create(n_pages: int) -> PagePool:
    return PagePool(n_pages)


def page_pool_alloc(pool: PagePool, n: int) -> np.ndarray:
    return pool.alloc(n)


def page_pool_free(pool: PagePool, ids) -> None:
    pool.free(ids)


def page_pool_free_count(pool: PagePool) -> int:
    return pool.free_count()


def page_pool_destroy(pool: PagePool) -> None:
    pool.close()


# ----------------------------------------------------------------------------- kernels

def _keep_alive(stream, *tensors) -> None:
    """Tensors allocated here on torch's current stream but used by kernels
    enqueued on another stream: tell the caching allocator, so their memory
    is not handed out again before that stream's work has finished."""
    if stream is None:
        return
    import torch
    if stream == torch.cuda.current_stream():
        return
    for t in tensors:
        t.record_stream(stream)


def write_kv(cache: KVCache, streams, k_new, v_new, stream=None) -> None:
    """Store bf16 rows [rows][Hkv][D] at each stream's positions first_pos.."""
    dev = []
    _v.cache(dev, cache, _v.any_paged(streams))
    rows = _v.streams(dev, cache, streams)
    if rows:
        _v.dense_rows(dev, "k_new", k_new, cache.n_kv_heads, cache.head_dim, rows)
        _v.dense_rows(dev, "v_new", v_new, cache.n_kv_heads, cache.head_dim, rows)
    _v.on_gpu(dev)
    arr, n = _streams(streams)
    cc = cache.c()
    _check(lib().write_kv(C.byref(cc), arr, n, _ptr(k_new), _ptr(v_new), _hip_stream(stream)),
           "write_kv")


def paged_attn_decode_workspace_size(streams, n_q_heads: int, head_dim: int,
                                     split_keys: int = DEFAULT_SPLIT_KEYS) -> int:
    arr, n = _streams(streams)
    return int(lib().paged_attn_decode_workspace_size(arr, n, int(n_q_heads), int(head_dim),
                                                      int(split_keys)))


def paged_attn_decode_plan(streams, n_q_heads: int, n_kv_heads: int, head_dim: int,
                           split_keys: int = DEFAULT_SPLIT_KEYS, kv_dtype: str = "bf16"):
    """(per-stream split counts, pa_decode_plan) without launching anything."""
    arr, n = _streams(streams)
    splits = np.zeros(max(n, 1), np.int32)
    plan = pa_decode_plan()
    _check(lib().paged_attn_decode_plan(arr, n, int(n_q_heads), int(n_kv_heads), int(head_dim),
                                        int(split_keys), _kv_code(kv_dtype),
                                        splits.ctypes.data_as(C.c_void_p),
                                        C.byref(plan)), "paged_attn_decode_plan")
    return splits[:n], plan


def _kv_code(kv_dtype: str) -> int:
    if kv_dtype == "bf16":
        return PA_KV_BF16
    if kv_dtype == "fp8":
        return PA_KV_FP8_E4M3
    raise ValueError(f"unknown KV dtype {kv_dtype!r}")


def _check_attention(dev: list, cache: KVCache, streams, q, out, max_rows=None) -> int:
    """Validate the tensors of an attention call (device checks are appended
    to `dev`, for _v.on_gpu once every other check has passed); returns
    n_q_heads."""
    if q is None and out is None:
        raise ValueError("q or out is required")
    ref = q if q is not None else out
    _v.cache(dev, cache, _v.any_paged(streams))
    rows = _v.streams(dev, cache, streams, max_rows)
    if not hasattr(ref, "shape") or len(ref.shape) != 3:
        raise ValueError("q / out must be [rows][n_q_heads][head_dim]")
    n_q_heads = int(ref.shape[1])
    if n_q_heads % cache.n_kv_heads:
        raise ValueError(f"{n_q_heads} q heads is not a multiple of {cache.n_kv_heads} kv heads")
    if q is not None:
        _v.dense_rows(dev, "q", q, n_q_heads, cache.head_dim, rows)
    if out is not None:
        _v.dense_rows(dev, "out", out, n_q_heads, cache.head_dim, rows)
    return n_q_heads


def paged_attn_decode(cache: KVCache, streams, q, out=None, sm_scale: float | None = None,
                      split_keys: int = DEFAULT_SPLIT_KEYS, workspace=None, stream=None):
    """Split-K decode; q/out bf16 [rows][Hq][D]. Returns out.

    A workspace or output allocated here on torch's current stream is marked
    as used by `stream`, so it cannot be reused while the kernels run there."""
    import torch
    dev = []
    n_q_heads = _check_attention(dev, cache, streams, q, out, DECODE_MAX_ROWS)
    made = []
    if out is None:
        out = torch.empty_like(q)
        made.append(out)
    if sm_scale is None:
        sm_scale = cache.head_dim ** -0.5
    arr, n = _streams(streams)
    need = int(lib().paged_attn_decode_workspace_size(arr, n, n_q_heads, cache.head_dim,
                                                      int(split_keys)))
    if workspace is None:
        _v.on_gpu(dev)
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
        made.append(workspace)
    else:
        _v.workspace(dev, workspace, need)
        _v.on_gpu(dev)
    cc = cache.c()
    _check(lib().paged_attn_decode(C.byref(cc), arr, n, _ptr(q), _ptr(out), n_q_heads,
                                   float(sm_scale), int(split_keys), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(),
                                   _hip_stream(stream)), "paged_attn_decode")
    _keep_alive(stream, *made)
    return out


def paged_attn_decode_noalloc(cache: KVCache, streams, q, out, sm_scale: float | None = None,
                              split_keys: int = DEFAULT_SPLIT_KEYS, stream=None):
    """Split-K decode with the partials in the library's fixed device scratch
    (no device allocation anywhere, so out must be given).  Calls that
    overlap on one GPU race on that scratch."""
    dev = []
    n_q_heads = _check_attention(dev, cache, streams, q, out, DECODE_MAX_ROWS)
    _v.on_gpu(dev)
    if sm_scale is None:
        sm_scale = cache.head_dim ** -0.5
    arr, n = _streams(streams)
    cc = cache.c()
    _check(lib().paged_attn_decode_noalloc(C.byref(cc), arr, n, _ptr(q), _ptr(out), n_q_heads,
                                           float(sm_scale), int(split_keys),
                                           _hip_stream(stream)), "paged_attn_decode_noalloc")
    return out


def hbm_read_probe(buf, sink, stream=None) -> None:
    """Stream-read the whole of device tensor buf (its bytes a multiple of 16)
    and fold it into sink (a one-element int32/uint32 device tensor): the
    reference read rate the attention kernels are measured against."""
    _v.on_gpu([("buf", buf), ("sink", sink)])
    nbytes = buf.numel() * buf.element_size()
    if not buf.is_contiguous() or sink.numel() < 1 or sink.element_size() != 4:
        raise ValueError("hbm_read_probe: buf must be contiguous and sink one 32-bit element")
    _check(lib().pa_hbm_read_probe(_ptr(buf), nbytes, _ptr(sink), _hip_stream(stream)),
           "pa_hbm_read_probe")


def decode_workspace(cache: KVCache, streams, n_q_heads: int,
                     split_keys: int = DEFAULT_SPLIT_KEYS, device="cuda"):
    """A device workspace tensor large enough for a decode call."""
    import torch
    nb = paged_attn_decode_workspace_size(streams, n_q_heads, cache.head_dim, split_keys)
    return torch.empty(max(nb, 256), dtype=torch.uint8, device=device)


def paged_attn_decode_partials(cache: KVCache, streams, q, workspace,
                               sm_scale: float | None = None,
                               split_keys: int = DEFAULT_SPLIT_KEYS, stream=None) -> None:
    """Split partials (m, l, o) of every (row, head, split) into workspace."""
    dev = []
    n_q_heads = _check_attention(dev, cache, streams, q, None, DECODE_MAX_ROWS)
    if sm_scale is None:
        sm_scale = cache.head_dim ** -0.5
    arr, n = _streams(streams)
    _v.workspace(dev, workspace, int(lib().paged_attn_decode_workspace_size(
        arr, n, n_q_heads, cache.head_dim, int(split_keys))))
    _v.on_gpu(dev)
    cc = cache.c()
    _check(lib().paged_attn_decode_partials(C.byref(cc), arr, n, _ptr(q), n_q_heads,
                                            float(sm_scale), int(split_keys), _ptr(workspace),
                                            workspace.numel() * workspace.element_size(),
                                            _hip_stream(stream)), "paged_attn_decode_partials")


def paged_attn_decode_merge(cache: KVCache, streams, out, workspace,
                            split_keys: int = DEFAULT_SPLIT_KEYS, stream=None):
    """Fixed-order LSE merge of the workspace partials into out (bf16)."""
    dev = []
    n_q_heads = _check_attention(dev, cache, streams, None, out, DECODE_MAX_ROWS)
    arr, n = _streams(streams)
    _v.workspace(dev, workspace, int(lib().paged_attn_decode_workspace_size(
        arr, n, n_q_heads, cache.head_dim, int(split_keys))))
    _v.on_gpu(dev)
    cc = cache.c()
    _check(lib().paged_attn_decode_merge(C.byref(cc), arr, n, _ptr(out), n_q_heads,
                                         int(split_keys), _ptr(workspace),
                                         workspace.numel() * workspace.element_size(),
                                         _hip_stream(stream)), "paged_attn_decode_merge")
    return out


def paged_attn_prefill(cache: KVCache, streams, q, out=None, sm_scale: float | None = None,
                       stream=None):
    """Causal prefill of every row of every stream; q/out bf16 [rows][Hq][D]."""
    import torch
    dev = []
    n_q_heads = _check_attention(dev, cache, streams, q, out)
    _v.on_gpu(dev)
    made = []
    if out is None:
        out = torch.empty_like(q)
        made.append(out)
    if sm_scale is None:
        sm_scale = cache.head_dim ** -0.5
    arr, n = _streams(streams)
    cc = cache.c()
    _check(lib().paged_attn_prefill(C.byref(cc), arr, n, _ptr(q), _ptr(out), n_q_heads,
                                    float(sm_scale), _hip_stream(stream)), "paged_attn_prefill")
    _keep_alive(stream, *made)
    return out
