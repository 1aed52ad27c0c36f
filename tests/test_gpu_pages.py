"""GPU tests of whole-page operations: copy on write of shared prefix pages,
multi-layer pools addressed through layer views, and page save / restore.
Every byte comparison is exact; attention results are compared with the
float64 oracle where the bytes alone do not settle it."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_addressing_amd as pa
import workloads
from tests._gpu import decode, launch_error, references, same_bytes, say
from tests._util import bits16

pytestmark = pytest.mark.gpu

HKV, D = 2, 128


def _rows(n, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    k = torch.randn((n, HKV, D), generator=g).to(torch.bfloat16)
    v = torch.randn((n, HKV, D), generator=g).to(torch.bfloat16)
    return k, v


def _bytes(t):
    return t.view(torch.uint8) if t.dtype == torch.uint8 else t.view(torch.int16)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_page_copy_moves_exactly_the_named_pages(dtype):
    cache = pa.alloc_pool(12, HKV, D, dtype)
    cache.k_scale = cache.v_scale = 0.01
    k, v = _rows(12 * 256, 3)
    pt = torch.arange(12, dtype=torch.int32, device="cuda")
    pa.write_kv(cache, [pa.Stream(12 * 256, 12 * 256, 0, 0, page_table=pt)], k.cuda(), v.cuda())
    k0, v0 = cache.k_pages.clone(), cache.v_pages.clone()
    src, dst = [1, 5, 0], [7, 2, 11]
    pa.page_copy(cache, src, dst)
    torch.cuda.synchronize()
    for p in range(12):
        want = src[dst.index(p)] if p in dst else p
        assert torch.equal(_bytes(cache.k_pages[p]), _bytes(k0[want])), p
        assert torch.equal(_bytes(cache.v_pages[p]), _bytes(v0[want])), p


def test_shared_prefix_with_copy_on_write_last_page():
    """Stream B shares stream A's full prefix pages, copies A's partial last
    page before writing its own rows there, and attends exactly as if it had
    stored the whole context itself; A is untouched."""
    pool = pa.PagePool(16)
    cache = pa.alloc_pool(16, HKV, D, "bf16")
    ctx_a = 3 * 256 + 100                     # 4 pages, the last one partial
    k, v = _rows(ctx_a + 40, 4)               # B = A's context + 40 own rows
    pages_a = pool.alloc(4)
    pt_a = torch.from_numpy(pages_a).cuda()
    pa.write_kv(cache, [pa.Stream(ctx_a, ctx_a, 0, 0, page_table=pt_a)], k[:ctx_a].cuda(),
                v[:ctx_a].cuda())
    g = torch.Generator("cpu").manual_seed(5)
    q = torch.randn((2, 8, D), generator=g).to(torch.bfloat16).cuda()
    st_a = pa.Stream(ctx_a, 1, 0, ctx_a - 1, page_table=pt_a)
    out_a = pa.paged_attn_decode(cache, [st_a], q)
    torch.cuda.synchronize()

    pool.share(pages_a[:3])                   # B takes A's three full pages
    own = pool.alloc(1)                       # and a page of its own for the partial one
    pa.page_copy(cache, [pages_a[3]], own)    # copy on write
    pages_b = np.concatenate([pages_a[:3], own])
    pt_b = torch.from_numpy(pages_b).cuda()
    ctx_b = ctx_a + 40
    pa.write_kv(cache, [pa.Stream(ctx_b, 40, 0, ctx_a, page_table=pt_b)], k[ctx_a:].cuda(),
                v[ctx_a:].cuda())
    st_b = pa.Stream(ctx_b, 1, 1, ctx_b - 1, page_table=pt_b)
    out_b = pa.paged_attn_decode(cache, [st_a, st_b], q)
    torch.cuda.synchronize()
    assert same_bytes(out_b[0], out_a[0])     # A unchanged by B's writes
    assert [pool.refcount(p) for p in pages_a] == [2, 2, 2, 1]

    # B against a private copy of everything: same bytes
    solo = pa.alloc_pool(16, HKV, D, "bf16")
    pt_s = torch.arange(4, dtype=torch.int32, device="cuda") + 9
    pa.write_kv(solo, [pa.Stream(ctx_b, ctx_b, 0, 0, page_table=pt_s)], k.cuda(), v.cuda())
    out_s = pa.paged_attn_decode(solo, [pa.Stream(ctx_b, 1, 1, ctx_b - 1, page_table=pt_s)], q)
    torch.cuda.synchronize()
    assert same_bytes(out_b[1], out_s[1])
    # and B's row against the oracle over its logical context (A's prefix rows
    # followed by B's own)
    kc = np.zeros((ctx_b, HKV, D), np.uint16)
    vc = np.zeros_like(kc)
    oracle.store(kc, vc, oracle.DTYPE_BF16, bits16(k), bits16(v), 0)
    ref = oracle.attention(kc, vc, oracle.DTYPE_BF16, bits16(q[1:2].cpu()), ctx_b - 1, HKV, ctx_b,
                           sm_scale=D ** -0.5)
    err = oracle.normalised_error(out_b[1:2].float().cpu().numpy(), ref)
    say(f"shared prefix: stream B error {err:.3e}")
    assert err <= 1e-2


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_multi_layer_pool_layer_views_equal_single_layer_pools(dtype):
    """A pool of [n_pages][L][Hkv][256][D] addressed one layer at a time (base
    advanced by the layer's block, page_stride spanning all L layers) gives
    each layer exactly the bytes and results of a pool of its own."""
    L, n_pages = 3, 9
    wl = workloads.build("layers", n_q_heads=8, n_kv_heads=HKV, head_dim=D, kv_dtype=dtype,
                         ctx_lens=[1500, 700], n_rows=[1, 3], n_pages=n_pages, seed=6)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.uint8
    vb = pa.v_block(dtype)
    k_all = torch.zeros((n_pages, L, HKV, 256, D), dtype=tdt, device="cuda")
    v_all = torch.zeros((n_pages, L, HKV, 256 // vb, D, vb), dtype=tdt, device="cuda")
    layer_stride = HKV * 256 * D
    outs = []
    for layer in range(L):
        view = pa.KVCache(k_all[:, layer], v_all[:, layer], n_pages, HKV, D, dtype,
                          wl.k_scale, wl.v_scale, page_stride=L * layer_stride)
        assert view.k_pages.data_ptr() == k_all.data_ptr() + layer * layer_stride * k_all.element_size()
        tables, streams = [], []
        for s, st in enumerate(wl.streams):
            pt = torch.from_numpy(st.pages).cuda()
            tables.append(pt)
            # each layer stores its own rows: the layer's rows are the stream's scaled copy
            kr = (wl.k_rows[s].float() * (layer + 1)).to(torch.bfloat16).cuda()
            vr = (wl.v_rows[s].float() * (layer + 1)).to(torch.bfloat16).cuda()
            pa.write_kv(view, [pa.Stream(st.ctx_len, st.ctx_len, 0, 0, page_table=pt)], kr, vr)
            streams.append(pa.Stream(st.ctx_len, st.n_rows, st.row_offset, st.first_pos,
                                     page_table=pt))
        q = wl.q.cuda()
        out = pa.paged_attn_decode(view, streams, q, sm_scale=wl.sm_scale)
        # the same layer in a pool of its own
        solo = pa.alloc_pool(n_pages, HKV, D, dtype)
        solo.k_scale, solo.v_scale = wl.k_scale, wl.v_scale
        for s, st in enumerate(wl.streams):
            kr = (wl.k_rows[s].float() * (layer + 1)).to(torch.bfloat16).cuda()
            vr = (wl.v_rows[s].float() * (layer + 1)).to(torch.bfloat16).cuda()
            pa.write_kv(solo, [pa.Stream(st.ctx_len, st.ctx_len, 0, 0, page_table=tables[s])],
                        kr, vr)
        out_solo = pa.paged_attn_decode(solo, streams, q, sm_scale=wl.sm_scale)
        torch.cuda.synchronize()
        assert torch.equal(_bytes(k_all[:, layer].contiguous()), _bytes(solo.k_pages))
        assert torch.equal(_bytes(v_all[:, layer].contiguous()), _bytes(solo.v_pages))
        assert same_bytes(out, out_solo)
        outs.append(out)
    assert not same_bytes(outs[0], outs[1])
    # layer 0 holds the workload's own rows: check it against the oracle
    refs, sels = references(wl)
    err = launch_error(wl, outs[0], refs, sels)
    say(f"multi-layer {dtype}: layer 0 error {err:.3e}")
    assert err <= (1e-2 if dtype == "bf16" else 3e-2)


def test_page_save_restore_round_trip():
    wl = workloads.build("save", n_q_heads=8, n_kv_heads=HKV, head_dim=D, kv_dtype="bf16",
                         ctx_lens=[1300], n_rows=[1], seed=7)
    from paged_kv_cache_addressing_amd.resident import upload
    res = upload(wl)
    before = decode(res)
    ids = wl.streams[0].pages
    nbytes = res.cache.k_pages[0].numel() * res.cache.k_pages.element_size()
    hk = torch.empty((len(ids), nbytes), dtype=torch.uint8, pin_memory=True)
    hv = torch.empty_like(hk, pin_memory=True)
    pa.page_save(res.cache, ids, hk, hv)
    torch.cuda.synchronize()
    for i, p in enumerate(ids):  # the host copy holds each page's bytes in order
        assert torch.equal(hk[i], res.cache.k_pages[p].cpu().view(torch.uint8).reshape(-1))
    res.cache.k_pages.zero_()
    res.cache.v_pages.zero_()
    pa.page_restore(res.cache, ids, hk, hv)
    torch.cuda.synchronize()
    assert same_bytes(decode(res), before)
