"""Host-side tensor checks of the Python binding: every kernel entry point
refuses a tensor that is too small, of the wrong dtype, strided where the
kernels assume dense rows, or not on the GPU, with ValueError and before
anything is launched.  Runs on the CPU: the checks run in the order dtype,
size, layout, device, so host tensors reach each of them."""
from __future__ import annotations

import pytest
import torch

import paged_kv_cache_addressing_amd as pa
from paged_kv_cache_addressing_amd import validate

HKV, D, HQ = 2, 128, 8


def pool(n_pages=4, dtype="bf16", extra=0):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.uint8
    n = n_pages * HKV * 256 * D + extra
    k = torch.zeros(n, dtype=tdt)
    v = torch.zeros(n, dtype=tdt)
    return pa.KVCache(k, v, n_pages, HKV, D, dtype)


def stream(ctx=600, rows=1, off=0, table_len=None, **kw):
    pt = torch.zeros(-(-ctx // 256) if table_len is None else table_len, dtype=torch.int32)
    return pa.Stream(ctx, rows, off, ctx - rows, page_table=pt, **kw)


def rows(n, heads=HQ, d=D, dtype=torch.bfloat16):
    return torch.zeros((n, heads, d), dtype=dtype)


def expect(fn, *a, match=None, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*a, **kw)


def test_host_tensors_reach_the_device_check_last():
    # everything well formed but on the host: only the device check is left
    expect(pa.paged_attn_prefill, pool(), [stream()], rows(1), match="GPU tensor")
    expect(pa.write_kv, pool(), [stream()], rows(1, HKV), rows(1, HKV), match="GPU tensor")


def test_q_and_out_checks():
    c, s = pool(), [stream(rows=3, off=2)]
    expect(pa.paged_attn_prefill, c, s, rows(4), match="rows")                # needs 5 rows
    expect(pa.paged_attn_prefill, c, s, rows(5, dtype=torch.float16), match="bfloat16")
    expect(pa.paged_attn_prefill, c, s, rows(5, d=64), match="head_dim")
    expect(pa.paged_attn_prefill, c, s, rows(5, heads=7), match="multiple")
    expect(pa.paged_attn_prefill, c, s, rows(5).transpose(0, 1).contiguous().transpose(0, 1),
           match="contiguous")
    expect(pa.paged_attn_prefill, c, s, rows(5), out=rows(4), match="rows")
    expect(pa.paged_attn_prefill, c, s, rows(5), out=rows(5, heads=4), match="shape")
    expect(pa.paged_attn_decode_merge, c, s, rows(4), torch.zeros(1 << 20, dtype=torch.uint8),
           match="rows")


def test_decode_rows_and_workspace_checks():
    c = pool()
    expect(pa.paged_attn_decode, c, [stream(ctx=600, rows=17)], rows(17), match="at most")
    s = [stream(ctx=600, rows=2)]
    need = pa.paged_attn_decode_workspace_size(s, HQ, D)
    small = torch.zeros(need - 1, dtype=torch.uint8)
    expect(pa.paged_attn_decode, c, s, rows(2), workspace=small, match="workspace")
    expect(pa.paged_attn_decode_partials, c, s, rows(2), small, match="workspace")
    expect(pa.paged_attn_decode_merge, c, s, rows(2), small, match="workspace")


def test_page_table_checks():
    c = pool()
    expect(pa.paged_attn_prefill, c, [stream(ctx=600, table_len=2)], rows(1), match="page_table")
    bad = stream()
    bad.page_table = bad.page_table.to(torch.int64)
    expect(pa.paged_attn_prefill, c, [bad], rows(1), match="int32")
    gap = stream()
    gap.page_table = torch.zeros(6, dtype=torch.int32)[::2]
    expect(pa.paged_attn_prefill, c, [gap], rows(1), match="contiguous")
    missing = stream()
    missing.page_table = None
    expect(pa.paged_attn_prefill, c, [missing], rows(1), match="page_table")


def test_pool_and_slab_extent_checks():
    # a pool one element short of n_pages * page_stride
    short = pool(extra=-1)
    expect(pa.paged_attn_prefill, short, [stream()], rows(1), match="k_pages")
    wrong = pool(dtype="fp8")
    wrong.dtype = "bf16"  # uint8 storage described as bf16
    expect(pa.paged_attn_prefill, wrong, [stream()], rows(1), match="bfloat16")
    # layer views: a strided view whose storage covers every page is accepted
    # up to the device check
    L = 3
    k_all = torch.zeros((4, L, HKV, 256, D), dtype=torch.bfloat16)
    view = pa.KVCache(k_all[:, 2], k_all[:, 2], 4, HKV, D, "bf16",
                      page_stride=L * HKV * 256 * D)
    expect(pa.paged_attn_prefill, view, [stream()], rows(1), match="GPU tensor")
    # the same view claiming one page more than the storage holds
    over = pa.KVCache(k_all[:, 2], k_all[:, 2], 5, HKV, D, "bf16",
                      page_stride=L * HKV * 256 * D)
    expect(pa.paged_attn_prefill, over, [stream()], rows(1), match="k_pages")
    ks = torch.zeros(HKV * 512 * D - 1, dtype=torch.bfloat16)
    vs = torch.zeros(HKV * 512 * D, dtype=torch.bfloat16)
    slab = pa.Stream(600, 1, 0, 599, k_slab=ks, v_slab=vs, slab_cap=512,
                     layout=pa.PA_LAYOUT_SLAB)
    expect(pa.paged_attn_prefill, pool(), [slab], rows(1), match="k_slab")


def test_tree_mask_and_store_checks():
    s = stream(ctx=600, rows=4, tree_mask=torch.zeros(3, dtype=torch.int32))
    expect(pa.paged_attn_prefill, pool(), [s], rows(4), match="tree_mask")
    s = stream(ctx=600, rows=4)
    expect(pa.write_kv, pool(), [s], rows(4, HQ), rows(4, HKV), match="shape")
    expect(pa.write_kv, pool(), [s], rows(3, HKV), rows(4, HKV), match="rows")


def test_page_save_restore_host_buffer_checks():
    c = pool()
    nb = HKV * 256 * D * 2
    hk = torch.zeros((2, nb), dtype=torch.uint8)
    expect(pa.page_save, c, [0, 1, 2], hk, hk, match="host_k")
    expect(pa.page_restore, c, [0, 1], hk[:, ::2], hk, match="host_k")


def test_extent_of_views():
    t = torch.zeros(100, dtype=torch.bfloat16)
    assert validate.extent_bytes(t) == 200
    assert validate.extent_bytes(t[10:]) == 180
    assert validate.extent_bytes(t[10:20]) == 180  # the storage past the view is addressable
