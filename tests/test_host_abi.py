"""Host-side tests of the C ABI: the library loads, exports every symbol the
header declares, the page pool behaves as documented, validation rejects bad
calls with the documented status before anything is launched, and the decode
plan is a function of each stream alone.  No GPU is touched."""
from __future__ import annotations

import ctypes as C
import math
import os
import re

import numpy as np
import pytest

import paged_kv_cache_addressing_amd as pa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # a non-null "device" address; never dereferenced on these paths


def declared_functions():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            names += re.findall(r"^PA_API\s+[\w\s\*]*?\b(\w+)\s*\(", text, re.M)
    return names


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 12
    lib = pa.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert set(pa.EXPORTS) == set(names)
    assert pa.lib().pa_version() >> 16 == 1


def test_hbm_read_probe_validation():
    L = pa.lib()
    sink = C.c_void_p(FAKE)
    for buf, nbytes, snk in ((None, 1024, sink), (C.c_void_p(FAKE), 1024, None),
                             (C.c_void_p(FAKE), 0, sink), (C.c_void_p(FAKE), 1000, sink),
                             (C.c_void_p(FAKE + 8), 1024, sink)):
        assert L.pa_hbm_read_probe(buf, nbytes, snk, None) == pa.PA_EINVAL


def test_every_kernel_launch_stub_is_defined():
    """Each kernel's host-side launch stub is defined in the library (a stub
    the host pass failed to emit would only show as a load error)."""
    import subprocess
    out = subprocess.run(["nm", "-D", "--undefined-only", pa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    assert "__device_stub__" not in out, out


def test_status_strings():
    for code in range(0, -8, -1):
        assert pa.status_string(code) and pa.status_string(code) != "unknown status"
    assert pa.status_string(-99) == "unknown status"


# ----------------------------------------------------------------------------- page pool

def test_pool_lowest_first_all_or_nothing():
    pool = pa.PagePool(10)
    assert pool.free_count() == 10
    a = pool.alloc(3)
    assert list(a) == [0, 1, 2]
    b = pool.alloc(4)
    assert list(b) == [3, 4, 5, 6]
    pool.free([1, 4])
    c = pool.alloc(3)
    assert list(c) == [1, 4, 7]
    assert pool.free_count() == 2
    with pytest.raises(pa.PagedAttnError) as e:
        pool.alloc(3)  # 2 free: refused, nothing claimed
    assert e.value.status == pa.PA_ENOSPC
    assert pool.free_count() == 2
    with pytest.raises(pa.PagedAttnError) as e:
        pool.alloc(11)  # can never fit
    assert e.value.status == pa.PA_ETOOBIG
    assert list(pool.alloc(2)) == [8, 9]
    assert pool.free_count() == 0
    assert len(pool.alloc(0)) == 0


def test_pool_free_rejects_bad_ids_atomically():
    pool = pa.PagePool(4)
    pool.alloc(2)
    for bad in ([2], [0, 0], [-1], [4], [0, 7]):
        with pytest.raises(pa.PagedAttnError) as e:
            pool.free(bad)
        assert e.value.status == pa.PA_ERANGE
    assert pool.free_count() == 2  # nothing was freed by the failed calls
    pool.free([0, 1])
    assert pool.free_count() == 4


def test_pool_shared_pages_count_references():
    pool = pa.PagePool(6)
    prefix = pool.alloc(3)              # stream A's pages
    assert [pool.refcount(i) for i in range(6)] == [1, 1, 1, 0, 0, 0]
    pool.share(prefix[:2])              # stream B reuses A's first two pages
    pool.share([prefix[0]])             # and stream C the first
    assert [pool.refcount(i) for i in prefix] == [3, 2, 1]
    pool.free(prefix)                   # A finishes: only its own third page is freed
    assert pool.free_count() == 4 and pool.refcount(prefix[2]) == 0
    assert list(pool.alloc(1)) == [2]   # lowest free id first
    pool.free([prefix[0], prefix[0]])   # two references dropped in one call
    assert pool.refcount(prefix[0]) == 0 and pool.refcount(prefix[1]) == 1
    for bad, status in (([prefix[1], prefix[1]], pa.PA_ERANGE),  # more than it holds
                        ([5], pa.PA_ERANGE), ([9], pa.PA_ERANGE)):
        with pytest.raises(pa.PagedAttnError) as e:
            pool.free(bad)
        assert e.value.status == status
    with pytest.raises(pa.PagedAttnError) as e:
        pool.share([4])                 # a free page cannot be shared
    assert e.value.status == pa.PA_ERANGE
    assert pool.refcount(prefix[1]) == 1  # the failed calls changed nothing
    with pytest.raises(pa.PagedAttnError):
        pool.refcount(6)


def test_page_copy_save_restore_validation():
    c = cache()
    ids = (C.c_int32 * 2)(0, 1)
    far = (C.c_int32 * 2)(0, 64)
    same = (C.c_int32 * 2)(2, 2)
    L = pa.lib()
    assert L.page_copy(None, ids, ids, 2, None) == pa.PA_EINVAL
    assert L.page_copy(C.byref(c), ids, far, 2, None) == pa.PA_ERANGE       # page 64 of 64
    assert L.page_copy(C.byref(c), ids, same, 2, None) == pa.PA_ERANGE      # two onto one
    assert L.page_copy(C.byref(c), ids, (C.c_int32 * 2)(1, 3), 2, None) == pa.PA_ERANGE  # dst is a src
    assert L.page_copy(C.byref(c), ids, ids, 0, None) == pa.PA_OK
    odd = cache(page_stride=4 * 256 * 256 + 1)  # not a multiple of 16 bytes
    assert L.page_copy(C.byref(odd), ids, (C.c_int32 * 2)(2, 3), 2, None) == pa.PA_EINVAL
    assert L.page_save(C.byref(c), far, 2, FAKE, FAKE, None) == pa.PA_ERANGE
    assert L.page_save(C.byref(c), ids, 2, None, FAKE, None) == pa.PA_EINVAL
    assert L.page_restore(C.byref(c), same, 2, FAKE, FAKE, None) == pa.PA_ERANGE
    assert L.page_restore(C.byref(c), ids, 2, FAKE, None, None) == pa.PA_EINVAL


def test_pool_create_rejects_empty():
    h = C.c_void_p()
    assert pa.lib().page_pool_create(0, C.byref(h)) == pa.PA_EINVAL
    assert pa.lib().page_pool_free_count(None) < 0


# ----------------------------------------------------------------------------- validation

def cache(**kw):
    c = pa.pa_kv_cache(FAKE, FAKE, 4 * 256 * 256, 64, 4, 256, pa.PA_KV_BF16, 1.0, 1.0)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def stream(**kw):
    s = pa.pa_stream(pa.PA_LAYOUT_PAGED, 1000, 1, 0, 999, 0, FAKE, None, None, 0)
    for k, v in kw.items():
        setattr(s, k, v)
    return s


def call_decode(c, ss, hq=24, scale=0.0625, split=4096, ws=FAKE, ws_bytes=1 << 30, q=FAKE):
    arr = (pa.pa_stream * len(ss))(*ss)
    return pa.lib().paged_attn_decode(C.byref(c) if c is not None else None, arr, len(ss), q,
                                      FAKE, hq, scale, split, ws, ws_bytes, None)


def call_prefill(c, ss, hq=24, scale=0.0625):
    arr = (pa.pa_stream * len(ss))(*ss)
    return pa.lib().paged_attn_prefill(C.byref(c), arr, len(ss), FAKE, FAKE, hq, scale, None)


def call_write(c, ss):
    arr = (pa.pa_stream * len(ss))(*ss)
    return pa.lib().write_kv(C.byref(c), arr, len(ss), FAKE, FAKE, None)


@pytest.mark.parametrize("fn", [call_prefill, call_write])
def test_validation_common(fn):
    assert fn(cache(dtype=5), [stream()]) == pa.PA_EINVAL
    assert fn(cache(head_dim=64, page_stride=4 * 256 * 64), [stream()]) == pa.PA_EUNSUPPORTED
    assert fn(cache(n_kv_heads=0), [stream()]) == pa.PA_EINVAL
    assert fn(cache(page_stride=100), [stream()]) == pa.PA_EINVAL
    assert fn(cache(k_pages=None), [stream()]) == pa.PA_EINVAL
    assert fn(cache(dtype=pa.PA_KV_FP8_E4M3, k_scale=0.0), [stream()]) == pa.PA_EINVAL
    assert fn(cache(dtype=pa.PA_KV_FP8_E4M3, v_scale=float("nan")), [stream()]) == pa.PA_EINVAL
    assert fn(cache(), [stream(first_pos=1000)]) == pa.PA_ERANGE  # row past the context
    assert fn(cache(), [stream(ctx_len=0, first_pos=0, n_rows=0)]) == pa.PA_EINVAL
    assert fn(cache(), [stream(layout=7)]) == pa.PA_EINVAL
    assert fn(cache(), [stream(reserved=1)]) == pa.PA_EINVAL
    assert fn(cache(), [stream(page_table=None)]) == pa.PA_EINVAL
    assert fn(cache(), [stream(layout=pa.PA_LAYOUT_SLAB, k_slab=FAKE, v_slab=FAKE,
                               slab_cap=1000)]) == pa.PA_EINVAL  # cap not a multiple of 256
    assert fn(cache(), [stream(layout=pa.PA_LAYOUT_SLAB, k_slab=FAKE, v_slab=None,
                               slab_cap=1024)]) == pa.PA_EINVAL
    two = [stream(n_rows=2, first_pos=998), stream(row_offset=1)]  # rows 0-1 and 1 overlap
    assert fn(cache(), two) == pa.PA_ERANGE
    # an ancestor table covers at most 32 rows (one 32-bit word each)
    assert fn(cache(), [stream(n_rows=33, first_pos=967, tree_mask=FAKE)]) == pa.PA_EINVAL
    assert fn(cache(), []) == pa.PA_OK  # nothing to do, nothing launched
    assert fn(cache(), [stream(n_rows=0)]) == pa.PA_OK


def test_validation_decode():
    assert call_decode(None, [stream()]) == pa.PA_EINVAL
    assert call_decode(cache(), [stream()], hq=23) == pa.PA_EINVAL  # Hq % Hkv
    assert call_decode(cache(), [stream()], scale=0.0) == pa.PA_EINVAL
    assert call_decode(cache(), [stream()], scale=float("inf")) == pa.PA_EINVAL
    assert call_decode(cache(), [stream()], split=1000) == pa.PA_EINVAL
    assert call_decode(cache(), [stream()], split=0) == pa.PA_EINVAL
    assert call_decode(cache(), [stream(n_rows=17, first_pos=983)]) == pa.PA_EINVAL
    assert call_decode(cache(), [stream()], ws=None) == pa.PA_EWORKSPACE
    assert call_decode(cache(), [stream()], ws_bytes=100) == pa.PA_EWORKSPACE
    assert call_decode(cache(), [stream()], ws=FAKE + 8) == pa.PA_EWORKSPACE  # misaligned
    assert call_decode(cache(), [stream()], q=None) == pa.PA_EINVAL


# ----------------------------------------------------------------------------- planning

def _plan(streams, hq=24, hkv=4, d=256, split=4096):
    return pa.paged_attn_decode_plan(streams, hq, hkv, d, split)


def test_decode_plan_decode_batch_shape():
    ss = [stream(ctx_len=65536, first_pos=65535, row_offset=i) for i in range(8)]
    splits, plan = _plan(ss)
    assert list(splits) == [16] * 8
    assert plan.total_splits == 128 and plan.col_tiles == 1
    # 512 one-split workgroups would take two rounds of the 256 CUs, so each
    # workgroup computes two consecutive splits of its stream
    assert plan.narrow_splits_per_wg == 2
    assert plan.partial_blocks == 256 and plan.merge_blocks == 8 * 24
    slots = 8 * 24 * 16
    want = math.ceil(slots * 256 * 4 / 256) * 256 + math.ceil(slots * 2 * 4 / 256) * 256
    assert plan.workspace_bytes == want == pa.paged_attn_decode_workspace_size(ss, 24, 256)


def test_decode_plan_verify_rows_and_ragged_lengths():
    lens = [4096, 4097, 8191, 110000, 4096 + 15]
    ss, off = [], 0
    for L in lens:
        ss.append(stream(ctx_len=L, n_rows=16, first_pos=L - 16, row_offset=off))
        off += 16
    splits, plan = _plan(ss)
    assert list(splits) == [math.ceil(L / 4096) for L in lens]
    # 16 rows x 6 q heads = 96 columns per kv head: one row-tile workgroup
    # per (split, kv head) covers them all; the streaming kernel runs none
    assert plan.col_tiles == 0
    assert plan.partial_blocks == plan.wide_blocks == sum(splits) * 4
    assert plan.narrow_splits_per_wg == 0


def test_decode_plan_kernel_choice_per_stream():
    # up to 32 (row, head) columns per kv head stream through registers
    # (one 16-column tile per workgroup); wider streams share LDS tiles
    ss = [stream(ctx_len=8192, n_rows=5, first_pos=8187, row_offset=0),
          stream(ctx_len=8192, n_rows=6, first_pos=8186, row_offset=5)]
    splits, plan = _plan(ss)
    assert list(splits) == [2, 2]
    assert plan.col_tiles == 2  # 30 columns
    assert plan.wide_blocks == 2 * 4
    assert plan.partial_blocks == 2 * 2 * 4 + 2 * 4
    assert plan.narrow_splits_per_wg == 1  # one round of workgroups: no grouping
    # head_dim 128: 48 columns a wave, 192 a workgroup; a group of 16 with
    # 16 rows (256 columns) needs two row tiles of 12 rows
    ss = [stream(ctx_len=4096, n_rows=16, first_pos=4080)]
    _, plan = pa.paged_attn_decode_plan(ss, 32, 2, 128, 4096)
    assert plan.wide_blocks == plan.partial_blocks == 2 * 2


def test_decode_plan_per_stream_independent_of_batch():
    a = stream(ctx_len=70000, n_rows=3, first_pos=69997)
    alone, _ = _plan([a])
    for others in ([stream(ctx_len=5000, first_pos=4999, row_offset=3)],
                   [stream(ctx_len=300000, n_rows=16, first_pos=299984, row_offset=3)]):
        batch, _ = _plan([a] + others)
        assert batch[0] == alone[0]


def test_decode_plan_groups_streams_beyond_one_launch():
    ss = [stream(ctx_len=512, first_pos=511, row_offset=i) for i in range(70)]
    splits, plan = _plan(ss)
    assert plan.n_launch_groups == 3  # 32 + 32 + 6
    assert plan.total_splits == 70 and plan.merge_blocks == 70 * 24
    empty = [stream(ctx_len=512, first_pos=511, row_offset=0, n_rows=0)]
    _, plan = _plan(empty)
    assert plan.n_launch_groups == 0 and plan.workspace_bytes == 0


def test_decode_plan_split_grouping_rule():
    """Consecutive splits share a register-streaming workgroup only once the
    one-split workgroups would take two or more rounds of 256 CUs, and only
    when a split's pages divide over the four waves (split_keys % 1024 == 0);
    the grouping is ceil(workgroups / 256)."""
    def batch(n, ctx):
        return [stream(ctx_len=ctx, first_pos=ctx - 1, row_offset=i) for i in range(n)]
    # 4 streams x 16 splits x 4 kv heads = 256 workgroups: one round, no grouping
    _, plan = _plan(batch(4, 65536))
    assert plan.narrow_splits_per_wg == 1 and plan.partial_blocks == 256
    # 12 streams: 768 one-split workgroups -> 3 splits each, 16 splits -> 6 per stream
    _, plan = _plan(batch(12, 65536))
    assert plan.narrow_splits_per_wg == 3 and plan.partial_blocks == 12 * 6 * 4
    # 512-key splits (two pages, not a multiple of four): never grouped
    _, plan = _plan(batch(8, 65536), split=512)
    assert plan.narrow_splits_per_wg == 1 and plan.partial_blocks == 8 * 128 * 4
    # 2,048-key splits: 8 x 32 x 4 = 1,024 workgroups -> 4 splits each
    _, plan = _plan(batch(8, 65536), split=2048)
    assert plan.narrow_splits_per_wg == 4 and plan.partial_blocks == 8 * 8 * 4
